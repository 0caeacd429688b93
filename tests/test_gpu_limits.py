"""The largest weights on either side of the split kernels' 32-bit weight
offsets (N*K < 2^32): just below the limit the split kernels run, at the limit
the projection is routed to the fp32 kernels (64-bit row offsets). Checked
through both routes (rtq_block_project's grouped launch and a single GEMM),
with a bias, on sampled output columns the oracle computes from the sampled
weight rows (rows are independent)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
K = 32768


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def big_weight(fmt, N, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if fmt == "q8":
        q = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
        scale = torch.rand(N, device=DEV, generator=g) * 0.01 + 1e-4
        return rtq.Q8Weight(q, scale)
    payload = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=DEV, generator=g)
    pairs = torch.empty((N, K // 32, 2), dtype=torch.float16, device=DEV)
    pairs[..., 0] = (torch.rand((N, K // 32), device=DEV, generator=g) * 0.01).half()
    pairs[..., 1] = (torch.rand((N, K // 32), device=DEV, generator=g) * -0.08).half()
    return rtq.Q4Weight(payload, pairs)


@pytest.mark.parametrize("fmt", ["q8", "q4"])
@pytest.mark.parametrize("N", [(1 << 32) // K - 1, (1 << 32) // K], ids=["below_2^32", "at_2^32"])
def test_weights_at_the_32bit_offset_limit(fmt, N):
    say(f"limits {fmt} N={N} K={K} (N*K = {N * K})")
    M = 3
    w = big_weight(fmt, N, 51 + N % 7)
    x = synth.activation(51, 0, "h", M, K)
    bias = (np.random.default_rng(52).standard_normal(N) * 0.1).astype(np.float32)
    xd = torch.from_numpy(x).to(DEV)
    bd = torch.from_numpy(bias).to(DEV)
    y_grouped = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    rtq.block_project([{"w1": rtq.Projection(w, xd, y_grouped, bd)}], M)
    y_single = rtq.gemm(xd, w)                       # rtq_gemm_q4 / _q8, no bias
    torch.cuda.synchronize()
    cols = np.sort(np.concatenate([np.random.default_rng(53).choice(N, 60, replace=False), [0, N - 1]]))
    ci = torch.as_tensor(cols, device=DEV)
    payload = w.payload[ci].cpu().numpy()
    scale = w.scale_tensor[ci].cpu().numpy()
    want = oracle.project(fmt, x, payload, scale)
    for y, b in ((y_grouped, bias[cols]), (y_single, 0.0)):
        err = oracle.rel_fro(y[:, ci].cpu().numpy(), want + np.asarray(b, dtype=np.float64))
        assert err <= 1e-5, err
    del w
    torch.cuda.empty_cache()
