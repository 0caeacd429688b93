"""GPU parity of the projection bias, y = x . W^T + b (b fp32 [N] added to
every row), in every arithmetic mode and on every route a projection can take:
the grouped small-M launch (bias added by the finish pass), the large-M tiles
(bias added in the epilogue) and the fp32 kernels (finish pass). Bars as for
the GEMM: rel. Frobenius 1e-5 against the oracle (3e-3 against fp32 x in the
bf16-activation mode, 1e-5 against its own bf16(x) reference)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MODES = {"split_bf16": rtq.MATH_SPLIT_BF16, "fp32_mfma": rtq.MATH_FP32_MFMA, "bf16": rtq.MATH_BF16,
         "split_f16": rtq.MATH_SPLIT_F16}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(params=list(MODES), ids=list(MODES))
def mode(request):
    """Arithmetic of the calls (its name; MODES gives the value passed to each call)."""
    return request.param


def bias_of(seed, N):
    return (synth.activation(seed, 0, "h", 1, N)[0] * 0.5).astype(np.float32)


def check(y, mode, fmt, x, ref, b):
    """Shapes the split kernels do not take (K not a multiple of 32) run on the
    fp32 kernels in every mode, at the fp32 bar."""
    if mode == "bf16" and x.shape[1] % 32 == 0:
        tight = oracle.rel_fro(y, oracle.project_bf16(fmt, x, *ref) + b.astype(np.float64)[None, :])
        assert tight <= 1e-5, tight
        err = oracle.rel_fro(y, oracle.project_bias(fmt, x, *ref, b))
        assert err <= 3e-3, err
    else:
        err = oracle.rel_fro(y, oracle.project_bias(fmt, x, *ref, b))
        assert err <= 1e-5, err


@pytest.mark.parametrize("M", [80, 333])
def test_block_project_with_biases(M, mode):
    """Every projection of two blocks, biases on all but wq of block 1 and w2
    of block 0, so biased and unbiased, chunked and unchunked projections mix."""
    say(f"bias block_project M={M} mode={mode}")
    blocks, refs = [], []
    for b in range(2):
        xs = {n: synth.activation(41, b, n, M) for n in synth.INPUT_WIDTH}
        dxs = {n: dev(v) for n, v in xs.items()}
        blk, ref = {}, {}
        for name in synth.PROJ_ORDER:
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(41, 0, b, name)
            fmt = rtq.RECIPE_MIXED[name]
            bias = None if (b, name) in ((1, "wq"), (0, "w2")) else bias_of(42 + b, N)
            blk[name] = rtq.Projection(rtq.quantize(dev(W), fmt), dxs[xin],
                                       torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV),
                                       None if bias is None else dev(bias))
            ref[name] = (fmt, oracle.quantize(W, fmt), xs[xin], bias)
        blocks.append(blk)
        refs.append(ref)
    rtq.block_project(blocks, M, math=MODES[mode])
    for b in range(2):
        for name, (fmt, r, x, bias) in refs[b].items():
            y = host(blocks[b][name].y)
            check(y, mode, fmt, x, r, np.zeros(y.shape[1], np.float32) if bias is None else bias)


@pytest.mark.parametrize("fmt,M,N,K", [("q4", 80, 512, 512), ("q8", 80, 512, 2048), ("f8", 17, 130, 96),
                                       ("q4", 300, 129, 64), ("q8", 33, 70, 33), ("f8", 129, 64, 40)])
def test_gemm_with_bias(fmt, M, N, K, mode):
    """Single projections, including shapes only the fp32 kernels take."""
    W = synth.weight(43, 0, 0, "w1", N, K, heavy="rows")
    x = synth.activation(43, 0, "x_ffn", M, K)
    b = bias_of(44, N)
    ref = oracle.quantize(W, fmt)
    y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), fmt), bias=dev(b), math=MODES[mode]))
    check(y, mode, fmt, x, ref, b)


@pytest.mark.parametrize("M", [80, 200])
def test_zero_weights_give_the_bias_exactly(M, mode):
    """W = 0 (int4 codes 0 with (scale, min) = (0, 0); int8 codes 0; FP8 code
    0): every output is exactly its column's bias."""
    N, K = 96, 512
    x = synth.activation(45, 0, "x_attn", M, K)
    b = bias_of(46, N)
    weights = [rtq.Q4Weight(dev(np.zeros((N, K // 2), np.uint8)), dev(np.zeros((N, K // 32, 2), np.float16))),
               rtq.Q8Weight(dev(np.zeros((N, K), np.int8)), dev(np.zeros(N, np.float32))),
               rtq.F8Weight(dev(np.zeros((N, K), np.uint8)))]
    for w in weights:
        y = host(rtq.gemm(dev(x), w, bias=dev(b), math=MODES[mode]))
        assert np.array_equal(y.view(np.uint32), np.broadcast_to(b, (M, N)).view(np.uint32)), type(w).__name__
