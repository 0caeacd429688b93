"""GPU tests of the activation range in every arithmetic and on every kernel
route: each row of x is scaled by its own power of two before the limb split
(and the output row scaled back), so rows from 1e-37 to 1e37 side by side,
zero rows and rows whose largest element dwarfs the rest each meet the bar.

Routes: M <= 32 with K in {256, 512, 1024, 2048} takes the direct small-M
kernel (row maxima found in the kernel), 33..80 the pre-pass and grouped
kernel, larger M the pre-pass and the tiled kernel; the fp32-MFMA arithmetic
takes its own kernels. The bf16-activation arithmetic is checked against the
oracle's bf16(x) GEMM on rows whose elements are all normal fp32 numbers (a
power-of-two scale does not change the rounding of those) and against fp32 x
at its 3e-3 bar on every row.
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
SHAPES = [("q4", 12, 96, 512), ("q8", 30, 64, 2048), ("f8", 20, 64, 1024), ("q4", 9, 40, 256),   # direct
          ("q4", 48, 96, 512), ("q8", 80, 64, 2048), ("f8", 40, 64, 512),                        # grouped
          ("q4", 200, 130, 512), ("q8", 160, 96, 1024)]                                           # tiled


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


def check_rows(y, x, fmt, ref, mode):
    want = oracle.project(fmt, x, *ref)
    nz = [i for i in range(x.shape[0]) if np.any(want[i] != 0)]
    errs = np.array([oracle.rel_fro(y[i], want[i]) for i in nz])
    worst = float(errs.max())
    say(f"  {mode}: worst row error {worst:.3e} (row {nz[int(np.argmax(errs))]})")
    if mode != "bf16":
        assert worst <= 1e-5, worst
        return
    assert worst <= 3e-3, worst
    want16 = oracle.project_bf16(fmt, x, *ref)
    tiny = np.finfo(np.float32).tiny
    normal = [i for i in nz if np.all((x[i] == 0) | (np.abs(x[i]) >= tiny))]
    assert normal, "no normal-range row"
    tight = max(oracle.rel_fro(y[i], want16[i]) for i in normal)
    assert tight <= 1e-5, tight


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("fmt,M,N,K", SHAPES)
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
@pytest.mark.parametrize("M", [1, 2])
def test_single_rows_at_the_ends_of_the_range(M, scale, mode):
    """One or two rows of the direct kernel at the top of the fp32 range, near
    its bottom, and made of subnormals (3e-39 is below 2^-126)."""
    K, N = 2048, 64
    say(f"single rows M={M} scale={scale} math={mode}")
    W = synth.weight(62, 0, 0, "w2", N, K)
    x = synth.activation(62, 0, "h", M, K).astype(np.float64)
    x = (x / np.abs(x).max(axis=1, keepdims=True) * scale).astype(np.float32)
    for fmt in ("q4", "q8"):
        ref = oracle.quantize(W, fmt)
        y = host(rtq.gemm(dev(x), rtq.quantize(dev(W), fmt), math=MODES[mode]))
        want = oracle.project(fmt, x, *ref)
        assert np.all(np.isfinite(y)), "row overflowed"
        if mode == "fp32" and scale < np.finfo(np.float32).tiny:
            # the fp32-MFMA arithmetic multiplies the unscaled x: products of
            # subnormal activations are themselves subnormal, so only the range
            # (no overflow, checked above) is asked of it here
            continue
        bar = 3e-3 if mode == "bf16" else 1e-5
        for i in range(M):
            e = oracle.rel_fro(y[i], want[i])
            assert e <= bar, (fmt, i, e)


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
