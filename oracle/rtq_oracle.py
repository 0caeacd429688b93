"""CPU oracle for the quantized-resident projection GEMM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, tables or constants with the HIP
library; the two receive the same seeded fp32 tensors and nothing else.

What is computed, and where the pages define it:

* Packed int4 weights (int4 model card "RT-J - int4 (Q4-style,
  mixed-precision) quantized checkpoints", section "Quantization format"):
  uint4 codes in groups of 32 along the input dimension, two codes per byte
  with the low nibble holding the even index, one fp16 (scale, min) pair per
  group, and W[o,i] ~ nibble * scale + min. Group ranges come from a min-MSE
  clip search over a shrink grid from 1.0 down to 0.8.
* Int8 weights (int8 model card "RT-J - int8 (Q8_0-style) quantized
  checkpoints", section "Quantization format"): one symmetric fp32 scale per
  output row, scale[o] = max|W[o,:]| / 127 and W[o,i] ~ q[o,i] * scale[o].
* The mixed recipe (int4 model card, same section): int4 for wq/wk/wv/wg and
  ffn.w1/w3, int8 for the residual-writing wo and ffn.w2.
* FP8 E4M3 weights (FP8 model card "RT-J - FP8 E4M3 checkpoints", section
  "FP8 Format"): each 2-D weight matrix is kept as PyTorch's
  float8_e4m3fn type with no companion scale, so W[o,i] is the E4M3 value of
  its one-byte code.
* The GEMM itself: y = x . W^T with the weights dequantized first (int4 model
  card, opening paragraph: the kernels dequantize inside the GEMM).
* The projection bias: the checkpoints keep biases in fp32 next to the
  quantized matrices (int4 model card, "Quantization format"), and a
  projection with a bias computes y = x . W^T + b, b[o] added to every row;
* The lower-precision variant of that GEMM with bf16 activations:
  y = bf16(x) . W^T, x rounded once to the nearest bfloat16 (the upper half of
  an IEEE binary32: 8 significant bits, the fp32 exponent range), ties to the
  even code, the IEEE 754 default rounding.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* payload layout u8[N, K/2] row-major; pair layout f16[N, K/32, 2] with
  [..., 0] = scale and [..., 1] = min;
* dequantized weights are fp32; the int4 form q*s+m and the int8 form q*scale
  are each exact in fp64, so computing them in fp64 and rounding once to fp32
  gives the single-rounded fp32 value;
* the GEMM reference is computed in fp64 from those fp32 weights;
* clip search: alpha in {1.00, 0.95, 0.90, 0.85, 0.80} (fp64 literals), both
  ends of the group range pulled toward zero: lo = alpha*min, hi = alpha*max;
  s16 = f16((hi - lo) / 15), m16 = f16(lo) rounded to nearest even from fp64;
  q = clip(rint((w - m16) / s16), 0, 15) (q = 0 when s16 == 0); the squared
  error sum_k ((q*s16 + m16) - w)^2 is accumulated in fp64 in index order with
  no fused operations; the first alpha with strictly smaller error wins, so
  ties keep the larger alpha;
* int8: q = clip(rint(w / scale), -127, 127) in fp64, q = 0 for a zero row;
* FP8: the code of an fp32 weight is what a cast to PyTorch's float8_e4m3fn
  gives: nearest E4M3 value, ties to the even code, NaN (with the input's
  sign) for magnitudes that round past 448, for infinities and for NaN.
"""
from __future__ import annotations

import numpy as np

GROUP = 32  # int4 group size along the input dimension
CLIP_GRID = (1.00, 0.95, 0.90, 0.85, 0.80)

# Format routing of the int4 card's mixed recipe, and of the all-int8 card.
RECIPE_MIXED = {"wq": "q4", "wk": "q4", "wv": "q4", "wg": "q4",
                "w1": "q4", "w3": "q4", "wo": "q8", "w2": "q8"}
RECIPE_ALL_Q8 = {name: "q8" for name in RECIPE_MIXED}
RECIPE_ALL_F8 = {name: "f8" for name in RECIPE_MIXED}   # FP8 card: every matrix weight


# ----------------------------------------------------------------------------
# Nibble packing (int4 card, "Quantization format": two nibbles per byte, the
# low nibble holds the even index).
# ----------------------------------------------------------------------------
def unpack_q4(payload: np.ndarray) -> np.ndarray:
    """u8[N, K/2] -> u8[N, K] nibble codes."""
    payload = np.asarray(payload, dtype=np.uint8)
    N, half = payload.shape
    q = np.empty((N, 2 * half), dtype=np.uint8)
    q[:, 0::2] = payload & 0x0F
    q[:, 1::2] = payload >> 4
    return q


def pack_q4(codes: np.ndarray) -> np.ndarray:
    """u8[N, K] codes in 0..15 -> u8[N, K/2] bytes."""
    codes = np.asarray(codes)
    if codes.shape[1] % 2:
        raise ValueError("K must be even to pack nibbles")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("nibble codes must lie in 0..15")
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


# ----------------------------------------------------------------------------
# Dequantization.
# ----------------------------------------------------------------------------
def dequant_q4(payload: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """W[o,i] = nibble * scale + min with one fp16 (scale, min) per 32-group.

    int4 card, "Quantization format". Returned as fp32: q*s+m is exact in fp64
    (q has 4 bits, s and m are fp16), so the fp64 value rounded to fp32 is the
    correctly rounded result.
    """
    q = unpack_q4(payload).astype(np.float64)
    N, K = q.shape
    pairs = np.asarray(pairs, dtype=np.float16).reshape(N, K // GROUP, 2)
    s = np.repeat(pairs[:, :, 0].astype(np.float64), GROUP, axis=1)
    m = np.repeat(pairs[:, :, 1].astype(np.float64), GROUP, axis=1)
    return (q * s + m).astype(np.float32)


def dequant_q8(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W[o,i] = q[o,i] * scale[o] (int8 card, "Quantization format").

    The product of an 8-bit integer and an fp32 scale is exact in fp64, so the
    cast to fp32 is the correctly rounded fp32 product.
    """
    q = np.asarray(q, dtype=np.int8).astype(np.float64)
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return (q * sc[:, None]).astype(np.float32)


# ----------------------------------------------------------------------------
# The contraction.
# ----------------------------------------------------------------------------
def gemm_ref(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y = x . W^T in fp64 from the fp32 operands (x [M,K], W [N,K])."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def project_q4(x, payload, pairs) -> np.ndarray:
    return gemm_ref(x, dequant_q4(payload, pairs))


def project_q8(x, q, scale) -> np.ndarray:
    return gemm_ref(x, dequant_q8(q, scale))


def rel_fro(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F (0 when both are zero)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ----------------------------------------------------------------------------
# Reference quantizers.
# ----------------------------------------------------------------------------
def _q4_candidate(w: np.ndarray, wmin: np.ndarray, wmax: np.ndarray, alpha: float):
    """One clip candidate for every group. w is fp64 [G, 32]."""
    lo = alpha * wmin
    hi = alpha * wmax
    s16 = ((hi - lo) / 15.0).astype(np.float16)
    m16 = lo.astype(np.float16)
    s = s16.astype(np.float64)
    m = m16.astype(np.float64)
    q = np.zeros(w.shape, dtype=np.float64)
    live = s > 0.0
    if live.any():
        r = np.rint((w[live] - m[live, None]) / s[live, None])
        q[live] = np.clip(r, 0.0, 15.0)
    err = np.zeros(w.shape[0], dtype=np.float64)
    for k in range(GROUP):                      # index order, one rounding per op
        recon = q[:, k] * s + m
        d = recon - w[:, k]
        sq = d * d
        err = err + sq
    return s16, m16, q, err


def quantize_q4(W: np.ndarray, return_alpha: bool = False):
    """fp32 W [N, K] -> (payload u8[N, K/2], pairs f16[N, K/32, 2]).

    Per 32-group min-MSE clip search over CLIP_GRID (int4 card,
    "Quantization format"). With return_alpha, also the chosen grid index per
    group, shape [N, K/32].
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 32 for int4 groups")
    G = K // GROUP
    w = W.astype(np.float64).reshape(N * G, GROUP)
    wmin = w.min(axis=1)
    wmax = w.max(axis=1)
    best = None
    for idx, alpha in enumerate(CLIP_GRID):
        s16, m16, q, err = _q4_candidate(w, wmin, wmax, alpha)
        if best is None:
            best = [s16, m16, q, err, np.zeros(N * G, dtype=np.int64)]
            continue
        take = err < best[3]
        best[0] = np.where(take, s16, best[0])
        best[1] = np.where(take, m16, best[1])
        best[2] = np.where(take[:, None], q, best[2])
        best[3] = np.where(take, err, best[3])
        best[4] = np.where(take, idx, best[4])
    s16, m16, q, _, alpha_idx = best
    codes = q.astype(np.uint8).reshape(N, K)
    pairs = np.stack([s16, m16], axis=1).astype(np.float16).reshape(N, G, 2)
    payload = pack_q4(codes)
    if return_alpha:
        return payload, pairs, alpha_idx.reshape(N, G)
    return payload, pairs


def quantize_q8(W: np.ndarray):
    """fp32 W [N, K] -> (q i8[N, K], scale f32[N]).

    scale[o] = max|W[o,:]| / 127 (int8 card, "Quantization format"), rounded
    once to fp32 (the fp64 quotient of an fp32 value by 127 never lies on an
    fp32 rounding midpoint, so this equals an fp32 division).
    """
    W = np.asarray(W, dtype=np.float32)
    amax = np.abs(W).max(axis=1).astype(np.float64)
    scale = (amax / 127.0).astype(np.float32)
    sc = scale.astype(np.float64)
    q = np.zeros(W.shape, dtype=np.float64)
    live = sc > 0.0
    q[live] = np.clip(np.rint(W[live].astype(np.float64) / sc[live, None]), -127.0, 127.0)
    return q.astype(np.int8), scale


# ----------------------------------------------------------------------------
# FP8 E4M3 weights (FP8 model card "RT-J - FP8 E4M3 checkpoints", section
# "FP8 Format": 2-D weight matrices are kept in PyTorch's float8_e4m3fn type
# and carry no scale). The E4M3 "fn" encoding: 1 sign bit, 4
# exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals
# m * 2^-9; there are no infinities, and S.1111.111 is NaN, so the largest
# finite magnitude is 1.75 * 2^8 = 448.
# ----------------------------------------------------------------------------
F8_NAN = 0x7F


def decode_f8(codes) -> np.ndarray:
    """u8 E4M3 codes -> their values in fp64 (exact), NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == F8_NAN, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def quantize_f8(W: np.ndarray) -> np.ndarray:
    """fp32 W -> u8 E4M3 codes, as a cast to PyTorch's float8_e4m3fn does it:
    the magnitude goes to the nearest point of the E4M3 grid, a tie to the
    point with the even code (even mantissa); a magnitude that rounds past 448
    (to the place 480 that code 0x7F would hold), an infinity and a NaN all
    become NaN (0x7F); the sign bit is the input's, -0 included."""
    w = np.asarray(W, dtype=np.float32).astype(np.float64)
    a = np.abs(w)
    grid = np.append(decode_f8(np.arange(F8_NAN, dtype=np.uint8)), 480.0)   # codes 0 .. 0x7F, ascending
    hi = np.clip(np.searchsorted(grid, np.nan_to_num(a, nan=np.inf), side="left"), 1, F8_NAN)
    lo = hi - 1
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(np.isnan(a) | (a > 480.0) | (code == F8_NAN), F8_NAN, code)
    sign = np.signbit(w).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def dequant_f8(codes) -> np.ndarray:
    """W[o,i] = the E4M3 value of its code, as fp32 (every E4M3 value is exact in fp32)."""
    return decode_f8(codes).astype(np.float32)


def project_f8(x, codes) -> np.ndarray:
    return gemm_ref(x, dequant_f8(codes))


# ----------------------------------------------------------------------------
# bf16 activations. A bfloat16 code is the upper 16 bits of a binary32:
# sign, 8 exponent bits (bias 127), 7 stored fraction bits; exponent 0 holds
# the subnormals m * 2^-133. The nearest bf16 of an fp32 value lies between the
# code that keeps its upper 16 bits (toward zero) and the next code away from
# zero; a tie goes to the even code, and past the largest finite value
# (2 - 2^-7) * 2^127 the next code is infinity, taken at its place 2^128.
# ----------------------------------------------------------------------------
def _bf16_magnitude(code) -> np.ndarray:
    """Magnitude of bf16 codes (no sign bit) in fp64; code 0x7F80 -> 2^128."""
    c = np.asarray(code, dtype=np.int64)
    e = (c >> 7) & 0xFF
    m = (c & 0x7F).astype(np.float64)
    return np.where(e == 0, m * 2.0 ** -133, (1.0 + m / 128.0) * np.exp2(e.astype(np.float64) - 127.0))


def round_bf16(x) -> np.ndarray:
    """fp32 x -> the nearest bf16 value (returned as fp32), ties to the even
    code; infinities and NaN pass through, the sign is kept."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.int64)
    sign = bits >> 31
    lo = (bits & 0x7FFFFFFF) >> 16          # toward zero
    hi = lo + 1                             # away from zero
    a = np.abs(x.astype(np.float64))
    finite = np.isfinite(x)
    lo_f, hi_f = np.where(finite, lo, 0), np.where(finite, hi, 1)
    d_lo = a - _bf16_magnitude(lo_f)
    d_hi = _bf16_magnitude(hi_f) - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi_f % 2 == 0)), hi_f, lo_f)
    out = ((sign << 15) | code) << 16
    out = out.astype(np.uint32).view(np.float32)
    return np.where(finite, out, x)


def project_bf16(fmt: str, x, payload, scale) -> np.ndarray:
    """y = bf16(x) . dequant(W)^T in fp64: the bf16-activation variant."""
    return project(fmt, round_bf16(x), payload, scale)


def project_bias(fmt: str, x, payload, scale, bias) -> np.ndarray:
    """y = x . dequant(W)^T + b in fp64, b[o] added to column o of every row."""
    y = project(fmt, x, payload, scale)
    return y + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]


def quantize(W: np.ndarray, fmt: str):
    """fp32 W -> (payload, scale): the scale companion is None for f8."""
    if fmt == "q4":
        return quantize_q4(W)
    if fmt == "q8":
        return quantize_q8(W)
    if fmt == "f8":
        return quantize_f8(W), None
    raise ValueError(f"unknown format {fmt!r}")


def dequant(fmt: str, payload, scale) -> np.ndarray:
    if fmt == "q4":
        return dequant_q4(payload, scale)
    if fmt == "q8":
        return dequant_q8(payload, scale)
    if fmt == "f8":
        return dequant_f8(payload)
    raise ValueError(f"unknown format {fmt!r}")


def project(fmt: str, x, payload, scale) -> np.ndarray:
    """y = x . dequant(W)^T in fp64."""
    return gemm_ref(x, dequant(fmt, payload, scale))
