"""GPU tests of the activation range in every arithmetic and on every kernel
route.

Routes that scale rows: the pre-pass (M > 32, or a K the direct kernel does not
take) scales each row of x by its own power of two before the limb split and
scales the output row back, so rows from 1e-37 to 1e37 side by side, zero rows
and rows whose largest element dwarfs the rest each meet the bar, in every
split arithmetic; the fp32-MFMA arithmetic multiplies the dequantized fp32
weights by the unscaled x, an fp32 GEMM's range. The direct small-M kernel
(M <= 32, K in {256, 512, 1024, 2048}) splits x unscaled: its documented band
is |x| in [2^-100, 2^100] for every element of a row, and a row far above it
overflows its code sums (pinned below: that row's outputs are not finite, the
other rows are unaffected).

The bf16-activation arithmetic is checked against the oracle's bf16 GEMM of
the row-scaled x (bf16(x * 2^e) * 2^-e, which is bf16(x) wherever x is a
normal fp32 number) at 1e-5 per row (its 3e-3 bar against fp32 x is a
whole-output bar on random data, checked elsewhere).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
import weight_only_quantized_rtq_amd as rtq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"split": rtq.MATH_SPLIT_BF16, "split16": rtq.MATH_SPLIT_F16, "bf16": rtq.MATH_BF16,
         "fp32": rtq.MATH_FP32_MFMA}
SCALED = [("q4", 48, 96, 512), ("q8", 80, 64, 2048), ("f8", 40, 64, 512),                        # grouped
          ("q4", 200, 130, 512), ("q8", 160, 96, 1024), ("q4", 12, 64, 96)]                       # tiled; K=96
DIRECT = [("q4", 12, 96, 512), ("q8", 30, 64, 2048), ("f8", 20, 64, 1024), ("q4", 9, 40, 256)]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def magnitude_rows(M, K, seed):
    x = synth.activation(seed, 0, "x_attn", M, K).astype(np.float64)
    exps = synth.uniform_ints(seed, (M,), -30, 30)
    x *= 10.0 ** exps[:, None]
    x[3] = 0.0
    x[5] *= 1e-6
    x[5, 7] = 3.0e4                                 # one element far above the rest of its row
    x[6] = x[1] / np.abs(x[1]).max() * 1e-37        # near the bottom of the normal fp32 range
    x[7] = x[2] / np.abs(x[2]).max() * 1e37         # near the top (outputs stay finite)
    x[M - 1] = 0.0
    return x.astype(np.float32)


def scaled_bf16_reference(fmt, x, ref):
    """y of the bf16-activation arithmetic: each row x_r rounded to bf16 after
    the exact power-of-two scale 2^e_r that puts its largest magnitude in
    [2^14, 2^15), and scaled back: bf16(x_r * 2^e_r) * 2^-e_r . W^T. For rows
    whose elements are normal fp32 numbers this is bf16(x_r) . W^T."""
    x64 = x.astype(np.float64)
    _, E = np.frexp(np.abs(x64).max(axis=1))
    e = 15 - E
    xs = np.ldexp(x64, e[:, None]).astype(np.float32)          # exact
    return np.ldexp(oracle.project_bf16(fmt, xs, *ref), -e[:, None])


def check_rows(y, x, fmt, ref, mode):
    want = oracle.project(fmt, x, *ref) if mode != "bf16" else scaled_bf16_reference(fmt, x, ref)
    nz = [i for i in range(x.shape[0]) if np.any(want[i] != 0)]
    errs = np.array([oracle.rel_fro(y[i], want[i]) for i in nz])
    worst = float(errs.max())
    say(f"  {mode}: worst row error {worst:.3e} (row {nz[int(np.argmax(errs))]})")
    assert worst <= 1e-5, worst


@pytest.mark.parametrize("mode,fmt,M,N,K", [(m, *c) for m in MODES for c in SCALED] +
                         [("fp32", *c) for c in DIRECT])
def test_rows_of_any_magnitude_each_meet_the_bar(fmt, M, N, K, mode):
    say(f"magnitudes {fmt} M={M} N={N} K={K} math={mode}")
    W = synth.weight(61, 0, 0, "wq", N, K, heavy="rows")
    ref = oracle.quantize(W, fmt)
    x = magnitude_rows(M, K, 61)
    y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), fmt), math=MODES[mode]))
    check_rows(y, x, fmt, ref, mode)
    assert np.all(y[3] == 0) and np.all(y[M - 1] == 0)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("scale", [1e37, 1e-37, 3e-39])
@pytest.mark.parametrize("M", [33, 130])
def test_single_rows_at_the_ends_of_the_range(M, scale, mode):
    """Rows at the top of the fp32 range, near its bottom, and made of
    subnormals (3e-39 is below 2^-126), on the grouped and the tiled route."""
    K, N = 2048, 64
    say(f"single rows M={M} scale={scale} math={mode}")
    W = synth.weight(62, 0, 0, "w2", N, K)
    x = synth.activation(62, 0, "h", M, K).astype(np.float64)
    x = (x / np.abs(x).max(axis=1, keepdims=True) * scale).astype(np.float32)
    for fmt in ("q4", "q8"):
        ref = oracle.quantize(W, fmt)
        y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), fmt), math=MODES[mode]))
        want = oracle.project(fmt, x, *ref) if mode != "bf16" else scaled_bf16_reference(fmt, x, ref)
        assert np.all(np.isfinite(y)), "row overflowed"
        if mode == "fp32" and scale < np.finfo(np.float32).tiny:
            # the fp32-MFMA arithmetic multiplies the unscaled x: products of
            # subnormal activations are themselves subnormal, so only the range
            # (no overflow, checked above) is asked of it here
            continue
        for i in range(M):
            e = oracle.rel_fro(y[i], want[i])
            assert e <= 1e-5, (fmt, i, e)


@pytest.mark.parametrize("mode", ["split", "split16", "bf16"])
@pytest.mark.parametrize("fmt,M,N,K", DIRECT)
def test_direct_kernel_range_band(fmt, M, N, K, mode):
    """The direct kernel's documented band: rows whose elements lie between
    2^-100 and 2^100 in magnitude (here 1e-30 .. 1e30, one row each side of
    the others) meet the bar row by row. A row at 1e37 lies far above it:
    its code sums may overflow, and then its outputs are not finite; they are
    never finite and wrong, and no other row is touched."""
    say(f"direct band {fmt} M={M} N={N} K={K} math={mode}")
    W = synth.weight(64, 0, 0, "wv", N, K)
    ref = oracle.quantize(W, fmt)
    x = synth.activation(64, 0, "x_attn", M, K).astype(np.float64)
    x *= 10.0 ** synth.uniform_ints(64, (M,), -25, 25)[:, None]
    x[1] = x[1] / np.abs(x[1]).max() * 1e30
    x[2] = x[2] / np.abs(x[2]).max() * 1e-30
    x = x.astype(np.float32)
    w = rtq.quantize(dev(W), fmt)
    y = host(rtq.gemm(dev(x), w, math=MODES[mode]))
    check_rows(y, x, fmt, ref, mode)
    xo = x.copy()
    xo[3] = (xo[3].astype(np.float64) / np.abs(xo[3]).max() * 1e37).astype(np.float32)
    yo = host(rtq.gemm(dev(xo), w, math=MODES[mode]))
    if np.all(np.isfinite(yo[3])):
        want = oracle.project(fmt, xo[3:4], *ref) if mode != "bf16" else scaled_bf16_reference(fmt, xo[3:4], ref)
        assert oracle.rel_fro(yo[3:4], want) <= 1e-5
    else:
        say("  the 1e37 row overflowed (documented)")
    keep = [i for i in range(M) if i != 3]
    assert np.array_equal(yo[keep].view(np.uint32), y[keep].view(np.uint32))


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("M", [16, 48, 200])
def test_nonfinite_row_stays_in_its_row(M, mode):
    K, N = 512, 64
    W = synth.weight(63, 0, 0, "wk", N, K)
    ref = oracle.quantize(W, "q4")
    x = synth.activation(63, 0, "x_attn", M, K)
    x[2, 100] = np.inf
    x[4, 9] = np.nan
    y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), "q4"), math=MODES[mode]))
    assert not np.any(np.isfinite(y[2])) and np.all(np.isnan(y[4]))
    keep = [i for i in range(M) if i not in (2, 4)]
    bar = 3e-3 if mode == "bf16" else 1e-5
    err = oracle.rel_fro(y[keep], oracle.project("q4", x[keep], *ref))
    assert err <= bar, err
