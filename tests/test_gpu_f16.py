"""GPU parity of the two-limb fp16 mode (RTQ_MATH_SPLIT_F16, passed to every call).

Each activation row is scaled by the power of two that puts its largest
magnitude in [2^14, 2^15) and split into two fp16 limbs, h = fp16(v) and
l = fp16(v - h): 22 significant bits of every element. The general parity
tests run this mode through their `math` fixture at the 1e-5 bar. These add
what is particular to it, against the CPU oracle (fp64) on the same seeded
inputs:
  * rows of very different magnitude in one call, each scaled on its own:
    every row meets the bar by itself;
  * rows of one to seventeen 512-wide pieces, and rows longer than the
    pre-pass keeps in registers (read twice);
  * a non-finite row stays in its row;
  * the small-M direct kernel runs the exact three-limb split in this mode;
  * on random data the 22-bit representation keeps the error near the fp32
    accumulation level: 2e-6, a tenth of the bar.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
MATH = rtq.MATH_SPLIT_F16          # the arithmetic every call below passes

TOL = 1e-5
TIGHT = 2e-6
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()




def row_errors(y, want):
    return [oracle.rel_fro(y[i], want[i]) for i in range(want.shape[0])]


@pytest.mark.parametrize("fmt,M,N,K", [("q4", 48, 96, 512), ("q8", 48, 64, 2048), ("f8", 40, 64, 512),
                                       ("q4", 200, 130, 512), ("q8", 160, 96, 1024)])
def test_rows_of_any_magnitude_each_meet_the_bar(fmt, M, N, K):
    """Magnitudes 1e-37 .. 1e37 side by side, zero rows, and rows whose
    largest element dwarfs the rest: each row takes its own exponent."""
    say(f"magnitudes {fmt} M={M} N={N} K={K}")
    W = synth.weight(41, 0, 0, "wq", N, K, heavy="rows")
    ref = oracle.quantize(W, fmt)
    x = synth.activation(41, 0, "x_attn", M, K).astype(np.float64)
    exps = synth.uniform_ints(M, (M,), -30, 30)
    x *= 10.0 ** exps[:, None]
    x[3] = 0.0
    x[5] *= 1e-6
    x[5, 7] = 3.0e4                                 # one element far above the rest of its row
    x[6] = x[1] / np.abs(x[1]).max() * 1e-37        # near the bottom of the normal fp32 range
    x[7] = x[2] / np.abs(x[2]).max() * 1e37         # near the top (outputs stay finite)
    x[M - 1] = 0.0
    x = x.astype(np.float32)
    w = rtq.quantize(dev(W), fmt)
    y = host(rtq.gemm(dev(x), w, math=MATH))
    want = oracle.project(fmt, x, *ref)
    nz = [i for i in range(M) if np.any(want[i] != 0)]
    errs = row_errors(y[nz], want[nz])
    say(f"  worst row error {max(errs):.3e} (row {nz[int(np.argmax(errs))]})")
    assert max(errs) <= TOL, max(errs)
    assert np.all(y[3] == 0) and np.all(y[M - 1] == 0)


@pytest.mark.parametrize("fmt,M,N,K", [("q4", 40, 64, 4096), ("q8", 40, 64, 2080), ("f8", 150, 64, 4096),
                                       ("q4", 150, 96, 2080), ("q4", 33, 32, 32), ("q8", 40, 32, 1536),
                                       ("f8", 200, 48, 1056), ("q4", 48, 32, 8320)])
def test_long_and_short_rows(fmt, M, N, K):
    """Rows of the pre-pass (one wave per row, 512-wide pieces): a single
    group (32), three pieces (1536), a last piece of one group (1056) or cut
    short (2080), rows above the four pieces it keeps in registers, read
    twice (4096, and 8320 with a seventeenth piece)."""
    say(f"long rows {fmt} M={M} N={N} K={K}")
    W = synth.weight(42, 0, 0, "w1", N, K)
    ref = oracle.quantize(W, fmt)
    x = synth.activation(42, 0, "x_ffn", M, K)
    w = rtq.quantize(dev(W), fmt)
    y = host(rtq.gemm(dev(x), w, math=MATH))
    err = oracle.rel_fro(y, oracle.project(fmt, x, *ref))
    assert err <= TOL, err


@pytest.mark.parametrize("M", [48, 200])
def test_nonfinite_row_stays_in_its_row(M):
    K, N = 512, 64
    W = synth.weight(43, 0, 0, "wk", N, K)
    ref = oracle.quantize(W, "q4")
    x = synth.activation(43, 0, "x_attn", M, K)
    x[2, 100] = np.inf
    x[4, 9] = np.nan
    w = rtq.quantize(dev(W), "q4")
    y = host(rtq.gemm(dev(x), w, math=MATH))
    assert not np.any(np.isfinite(y[2])) and np.all(np.isnan(y[4]))
    keep = [i for i in range(M) if i not in (2, 4)]
    err = oracle.rel_fro(y[keep], oracle.project("q4", x[keep], *ref))
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", ["q4", "q8", "f8"])
def test_small_m_runs_the_exact_direct_split(fmt):
    """M <= 32 with K in 256..2048 takes the direct kernel, which needs no
    row scale and runs the three-limb split: bit for bit the output of
    RTQ_MATH_SPLIT_BF16."""
    M, N, K = 16, 128, 512
    W = synth.weight(44, 0, 0, "wv", N, K)
    x = dev(synth.activation(44, 0, "x_attn", M, K))
    w = rtq.quantize(dev(W), fmt)
    y16 = host(rtq.gemm(x, w, math=MATH)).copy()
    y3 = host(rtq.gemm(x, w, math=rtq.MATH_SPLIT_BF16))
    assert np.array_equal(y16.view(np.uint32), y3.view(np.uint32))


@pytest.mark.parametrize("fmt,M,N,K", [("q4", 80, 512, 512), ("q8", 80, 512, 2048), ("f8", 80, 512, 512),
                                       ("q4", 1000, 256, 512), ("q8", 1000, 256, 2048)])
def test_random_data_error_is_near_fp32_accumulation(fmt, M, N, K):
    say(f"tight {fmt} M={M} N={N} K={K}")
    W = synth.weight(45, 0, 0, "w3", N, K)
    ref = oracle.quantize(W, fmt)
    x = synth.activation(45, 0, "x_ffn", M, K)
    w = rtq.quantize(dev(W), fmt)
    xd = dev(x)
    y16 = host(rtq.gemm(xd, w, math=MATH)).copy()
    want = oracle.project(fmt, x, *ref)
    e16 = oracle.rel_fro(y16, want)
    e3 = oracle.rel_fro(host(rtq.gemm(xd, w, math=rtq.MATH_SPLIT_BF16)), want)
    say(f"  split_f16 {e16:.3e}  split_bf16 {e3:.3e}")
    assert e16 <= TIGHT, e16


def test_block_project_twelve_blocks_m80():
    """The grouped launch over 96 projections (w2's K chunks summed by the
    finish pass) in this mode, every output against the oracle."""
    cfg = 46
    M = 80
    projs, refs = [], []
    for b in range(12):
        blk, xs = {}, {}
        for name in synth.PROJ_ORDER:
            fmt = oracle.RECIPE_MIXED[name]
            N, K, xin = synth.BLOCK_SHAPES[name]
            W = synth.weight(cfg, 0, b, name)
            if xin not in xs:
                x = synth.activation(cfg, b, xin, M)
                xs[xin] = (x, dev(x))
            x, xd = xs[xin]
            blk[name] = rtq.Projection(weight=rtq.quantize(dev(W), fmt), x=xd,
                                       y=torch.empty(M, N, dtype=torch.float32, device=DEV))
            refs.append((b, name, fmt, x, oracle.quantize(W, fmt)))
        projs.append(blk)
    rtq.block_project(projs, M, math=MATH)
    for b, name, fmt, x, packed in refs:
        err = oracle.rel_fro(host(projs[b][name].y), oracle.project(fmt, x, *packed))
        assert err <= TOL, (b, name, err)
