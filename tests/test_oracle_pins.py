"""Pins for the CPU oracle: it is checked against what the pages and the
mathematics fix, never against itself.

Each pin_* function takes an oracle-like namespace, so the same pins also run
against deliberately broken copies of oracle functions (planted on the CPU, at
the bottom of this file) to show that a plausible mistake - a swapped nibble, a
dropped term, a transposed operand, an off-by-one - fails at least one pin.
"""
from __future__ import annotations

import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.exact import BF16, F16, F32, rint_half_even, round_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


def _f16_from_bits(rng, n, lo_exp=-10, hi_exp=4):
    """Random finite fp16 values with exponents in [lo_exp, hi_exp], both signs."""
    e = rng.integers(lo_exp, hi_exp + 1, size=n)
    frac = rng.integers(0, 1024, size=n)
    sign = rng.integers(0, 2, size=n)
    bits = (sign << 15) | ((e + 15) << 10) | frac
    return bits.astype(np.uint16).view(np.float16)


# ----------------------------------------------------------------------------
# Pins. Each raises AssertionError (or any exception) on a wrong oracle.
# ----------------------------------------------------------------------------
def pin_nibble_golden(o):
    for line in _rows("nibble_order.txt"):
        b, even, odd = line.split()
        byte = np.array([[int(b, 16)]], dtype=np.uint8)
        codes = o.unpack_q4(byte)
        assert codes.tolist() == [[int(even), int(odd)]], (b, codes)
        assert o.pack_q4(np.array([[int(even), int(odd)]])).tolist() == [[int(b, 16)]]


def pin_pack_roundtrip(o):
    allbytes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    assert np.array_equal(o.pack_q4(o.unpack_q4(allbytes)), allbytes)
    a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    pairs = np.stack([a.ravel(), b.ravel()], axis=1)            # [256, 2] codes
    assert np.array_equal(o.unpack_q4(o.pack_q4(pairs)), pairs)
    # a longer row keeps order across bytes: codes 0..15,15..0
    row = np.concatenate([np.arange(16), np.arange(15, -1, -1)])[None, :]
    assert np.array_equal(o.unpack_q4(o.pack_q4(row)), row)


def pin_q4_dequant_golden(o):
    for line in _rows("q4_dequant_examples.txt"):
        b, s, m, w0, w1 = line.split()
        payload = np.zeros((1, 16), dtype=np.uint8)
        payload[0, 0] = int(b, 16)
        pairs = np.array([[[float(s), float(m)]]], dtype=np.float16)
        W = o.dequant_q4(payload, pairs)
        assert W.dtype == np.float32 and W.shape == (1, 32)
        assert W[0, 0] == np.float32(w0) and W[0, 1] == np.float32(w1), (line, W[0, :2])
        assert np.all(W[0, 2:] == np.float32(m))                 # zero bytes give the min


def pin_q4_dequant_identity_probe(o):
    rng = np.random.default_rng(1)
    payload = rng.integers(0, 256, size=(5, 48), dtype=np.uint8)   # K = 96, 3 groups
    pairs = np.zeros((5, 3, 2), dtype=np.float16)
    pairs[..., 0] = 1.0
    W = o.dequant_q4(payload, pairs)
    assert np.array_equal(W, o.unpack_q4(payload).astype(np.float32))


def pin_q4_dequant_rational(o):
    rng = np.random.default_rng(2)
    N, K = 3, 64
    payload = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    pairs = np.stack([_f16_from_bits(rng, N * 2), _f16_from_bits(rng, N * 2)], axis=1).reshape(N, 2, 2)
    W = o.dequant_q4(payload, pairs)
    for n in range(N):
        for j in range(K // 2):
            byte = int(payload[n, j])
            for k, code in ((2 * j, byte & 15), (2 * j + 1, byte >> 4)):
                s = Fraction(float(pairs[n, k // 32, 0]))
                m = Fraction(float(pairs[n, k // 32, 1]))
                want = round_rne(code * s + m, F32)
                assert float(W[n, k]) == want, (n, k, float(W[n, k]), want)


def pin_q8_dequant_rational(o):
    rng = np.random.default_rng(3)
    N, K = 4, 40
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    scale = (rng.standard_normal(N) * 0.01).astype(np.float32)
    W = o.dequant_q8(q, scale)
    for n in range(N):
        for k in range(K):
            want = round_rne(Fraction(int(q[n, k])) * Fraction(float(scale[n])), F32)
            assert float(W[n, k]) == want


def pin_q8_golden(o):
    for line in _rows("q8_examples.txt"):
        vals, sc, qs = [p.split() for p in line.split(";")]
        W = np.array([[float(v) for v in vals]], dtype=np.float32)
        q, scale = o.quantize_q8(W)
        assert scale.dtype == np.float32 and q.dtype == np.int8
        assert float(scale[0]) == float(sc[0]), (line, scale)
        assert q[0].tolist() == [int(v) for v in qs], (line, q)


def pin_q8_closed_form(o):
    W = synth.weight(0, 0, 0, "wo", 24, 96, heavy="rows")
    W[3, :] = 0.0                                               # an all-zero row
    q, scale = o.quantize_q8(W)
    for n in range(W.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in W[n])
        want = round_rne(amax / 127, F32)
        assert float(scale[n]) == want, (n, float(scale[n]), want)
        if want == 0.0:
            assert not q[n].any()
            continue
        arg = int(np.argmax(np.abs(W[n])))
        assert int(q[n, arg]) == (127 if W[n, arg] > 0 else -127)
        sc = Fraction(want)
        for k in range(W.shape[1]):
            assert -127 <= int(q[n, k]) <= 127
            err = abs(int(q[n, k]) * sc - Fraction(float(W[n, k])))
            assert err <= sc * (Fraction(1, 2) + Fraction(1, 2**40)), (n, k)
            # the code is the nearest integer to w/scale (ties to even)
            assert int(q[n, k]) == max(-127, min(127, rint_half_even(Fraction(float(W[n, k])) / sc)))


def pin_q4_recon_bound(o):
    W = synth.weight(0, 0, 0, "wq", 8, 128, heavy="cols")
    payload, pairs = o.quantize_q4(W)
    codes = o.unpack_q4(payload)
    checked = 0
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            s = Fraction(float(pairs[n, k // 32, 0]))
            m = Fraction(float(pairs[n, k // 32, 1]))
            w = Fraction(float(W[n, k]))
            assert 0 <= int(codes[n, k]) <= 15
            if s > 0 and m <= w <= m + 15 * s:
                err = abs(int(codes[n, k]) * s + m - w)
                assert err <= s * (Fraction(1, 2) + Fraction(1, 2**40)), (n, k, float(err), float(s))
                checked += 1
    assert checked > 0.8 * W.size


def pin_q4_grid_roundtrip(o):
    """Weights already on a 16-level grid with fp16 (s, m) come back exactly,
    with alpha = 1.0 chosen and zero reconstruction error."""
    rng = np.random.default_rng(4)
    N, G = 6, 4
    s = (2.0 ** rng.integers(-8, -4, size=(N, G))) * rng.integers(1, 8, size=(N, G))
    m = -(2.0 ** rng.integers(-6, -2, size=(N, G))) * rng.integers(1, 4, size=(N, G))
    codes = rng.integers(0, 16, size=(N, G, 32))
    codes[..., 0] = 0
    codes[..., 1] = 15
    Wexact = codes * s[..., None] + m[..., None]
    W = Wexact.reshape(N, G * 32).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), Wexact.reshape(N, G * 32))  # exact in fp32
    payload, pairs, alpha = o.quantize_q4(W, return_alpha=True)
    assert np.all(alpha == 0)
    assert np.array_equal(pairs[..., 0].astype(np.float64), s)
    assert np.array_equal(pairs[..., 1].astype(np.float64), m)
    assert np.array_equal(o.unpack_q4(payload), codes.reshape(N, G * 32))
    assert np.array_equal(o.dequant_q4(payload, pairs), W)


def _brute_alpha(w32):
    """Independent clip search for one group: pure Python, exact-rational MSE."""
    wmin, wmax = min(w32), max(w32)
    best, best_err = None, None
    for idx, alpha in enumerate((1.00, 0.95, 0.90, 0.85, 0.80)):
        lo, hi = alpha * wmin, alpha * wmax
        s16 = round_rne(Fraction((hi - lo) / 15.0), F16)
        m16 = round_rne(Fraction(lo), F16)
        err = Fraction(0)
        for w in w32:
            q = 0 if s16 <= 0 else max(0, min(15, round((w - m16) / s16)))
            err += (q * Fraction(s16) + Fraction(m16) - Fraction(w)) ** 2
        if best_err is None or err < best_err:
            best, best_err = idx, err
    return best


def pin_q4_clip_argmin(o):
    W = np.concatenate([synth.weight(0, 0, 0, "w1", 6, 64),
                        synth.weight(0, 0, 0, "w3", 6, 64, heavy="cols")], axis=0)
    _, _, alpha = o.quantize_q4(W, return_alpha=True)
    for n in range(W.shape[0]):
        for g in range(W.shape[1] // 32):
            w32 = [float(v) for v in W[n, 32 * g:32 * g + 32]]
            assert int(alpha[n, g]) == _brute_alpha(w32), (n, g)


def pin_q4_degenerate(o):
    W = np.zeros((3, 64), dtype=np.float32)
    W[1, :32] = 0.3
    W[2, 32:] = -1.5
    payload, pairs = o.quantize_q4(W)
    assert not o.unpack_q4(payload).any()
    assert np.all(pairs[..., 0] == 0)
    assert pairs[1, 0, 1] == np.float16(0.3) and pairs[2, 1, 1] == np.float16(-1.5)
    assert np.array_equal(o.dequant_q4(payload, pairs)[0], np.zeros(64, np.float32))


def _loop_gemm(x, W):
    M, K = x.shape
    N = W.shape[0]
    y = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(x[i, k]) * float(W[j, k])
            y[i][j] = acc
    return np.array(y)


def pin_gemm_triple_loop(o):
    for (M, N, K) in ((1, 1, 32), (3, 5, 64), (7, 9, 96), (4, 4, 32)):
        g = np.random.default_rng(M * 100 + N)
        x = g.standard_normal((M, K)).astype(np.float32)
        W = g.standard_normal((N, K)).astype(np.float32)
        y = o.gemm_ref(x, W)
        assert y.shape == (M, N)
        ref = _loop_gemm(x, W)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12), (M, N, K)


def pin_gemm_exact_integer(o):
    """Integer x and dyadic dequantized weights: every product and sum is exact,
    so the projection equals integer arithmetic exactly."""
    M, N, K = 5, 7, 64
    x = synth.uniform_ints(1, (M, K), -4, 4).astype(np.float32)
    payload = synth.uniform_bytes(2, (N, K // 2))
    pairs = np.zeros((N, K // 32, 2), dtype=np.float16)
    pairs[..., 0] = 0.25
    pairs[..., 1] = -2.0
    y = o.project_q4(x, payload, pairs)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                byte = int(payload[j, k // 2])
                code = byte & 15 if k % 2 == 0 else byte >> 4
                acc += int(x[i, k]) * (Fraction(code, 4) - 2)
            assert Fraction(float(y[i, j])) == acc, (i, j)


# ---- FP8 E4M3 (FP8 model card, "FP8 Format": float8_e4m3fn weights, no scale) ----
def _f8_value(code):
    """The E4M3 value of a code from its bit fields, exactly; None for NaN."""
    if code & 0x7F == 0x7F:
        return None
    e, m = (code >> 3) & 0xF, code & 0x7
    mag = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if code & 0x80 else mag


def pin_f8_golden(o):
    for line in _rows("f8_examples.txt"):
        kind, rest = line.split(" ", 1)
        a, b = (t.strip() for t in rest.split(";"))
        if kind == "decode":
            v = float(o.decode_f8(np.array([int(a, 16)], dtype=np.uint8))[0])
            if b == "nan":
                assert math.isnan(v), line
            else:
                assert v == float(b) and math.copysign(1.0, v) == math.copysign(1.0, float(b)), line
        else:
            code = int(o.quantize_f8(np.array([float(a)], dtype=np.float32))[0])
            assert code == int(b, 16), (line, hex(code))


def pin_f8_decode_rational(o):
    vals = o.decode_f8(np.arange(256, dtype=np.uint8))
    for c in range(256):
        ref = _f8_value(c)
        if ref is None:
            assert math.isnan(vals[c]), c
        else:
            assert Fraction(float(vals[c])) == ref, c
            if c & 0x80:
                assert math.copysign(1.0, float(vals[c])) < 0, c


def pin_f8_roundtrip(o):
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = o.decode_f8(codes).astype(np.float32)
    assert np.array_equal(o.quantize_f8(vals), codes)


def pin_f8_nearest(o):
    """Brute force: the code is the nearest E4M3 value, ties to the even code,
    NaN past the 448/480 midpoint, the sign bit always the input's."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(600) * 10.0 ** rng.integers(-4, 3, 600)).astype(np.float32)
    mids = [(_f8_value(c) + _f8_value(c + 1)) / 2 for c in range(0, 126, 7)]
    w = np.concatenate([w, np.array([float(m) for m in mids] + [-float(m) for m in mids], dtype=np.float32)])
    got = o.quantize_f8(w)
    grid = [(c, _f8_value(c)) for c in range(127)] + [(0x7F, Fraction(480))]
    for x, code in zip(w.tolist(), got.tolist()):
        ax = abs(Fraction(x))
        best = min(grid, key=lambda cv: (abs(cv[1] - ax), cv[0] % 2))[0]
        if best == 0x7F or ax > 480:
            best = 0x7F
        assert code == best | (0x80 if math.copysign(1.0, x) < 0 else 0), (x, hex(code), hex(best))


PINS_F8 = [pin_f8_golden, pin_f8_decode_rational, pin_f8_roundtrip, pin_f8_nearest]


# ---- bf16 activations (the lower-precision variant y = bf16(x) . W^T) ----
def _bits(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def pin_bf16_golden(o):
    for line in _rows("bf16_examples.txt"):
        a, b = (int(t.strip(), 16) for t in line.split(";"))
        x = np.array([a], dtype=np.uint32).view(np.float32)
        got = _bits(o.round_bf16(x)[0])
        assert got == b, (line, hex(got))


def pin_bf16_nearest(o):
    """Exact rational rounding (IEEE definition on Fractions) of random fp32
    values over the whole exponent range, and of constructed midpoints."""
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 2 ** 32, size=3000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]                     # finite only
    mids = (rng.integers(0, 2 ** 16, size=400, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    mids = mids[((mids >> 23) & 0xFF) != 0xFF]
    x = np.concatenate([bits, mids]).view(np.float32)
    got = o.round_bf16(x)
    for v, g in zip(x.tolist(), got.tolist()):
        ref = round_rne(Fraction(v), BF16)
        assert g == ref and math.copysign(1.0, g) == math.copysign(1.0, v), (v, g, ref)


def pin_project_bf16(o):
    """y = bf16(x) . W^T: a triple loop over the exactly rounded x (Fraction
    rounding, not the oracle's), with the weights of the int8 closed form."""
    rng = np.random.default_rng(19)
    x = rng.standard_normal((3, 40)).astype(np.float32)
    q = rng.integers(-127, 128, size=(5, 40)).astype(np.int8)
    scale = (rng.random(5) * 0.01 + 0.001).astype(np.float32)
    xr = np.array([[round_rne(Fraction(float(v)), BF16) for v in row] for row in x])
    # the int8 closed form, single-rounded to fp32 (each q*scale is exact in fp64)
    W = (q.astype(np.float64) * scale.astype(np.float64)[:, None]).astype(np.float32).astype(np.float64)
    ref = _loop_gemm(xr, W)
    got = o.project_bf16("q8", x, q, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=0), np.abs(got - ref).max()
    assert not np.allclose(got, _loop_gemm(x.astype(np.float64), W), rtol=1e-6, atol=0)


PINS_BF16 = [pin_bf16_golden, pin_bf16_nearest, pin_project_bf16]


def pin_project_bias(o):
    """y = x . W^T + b: a triple loop with the bias added per output column, on
    an exactly representable case (small integers), and b alone for x = 0."""
    rng = np.random.default_rng(29)
    x = rng.integers(-3, 4, size=(4, 64)).astype(np.float32)
    payload = rng.integers(0, 256, size=(6, 32), dtype=np.uint8)
    pairs = np.zeros((6, 2, 2), dtype=np.float16)
    pairs[..., 0] = 0.5
    pairs[..., 1] = -4.0
    bias = np.array([0.25, -1.5, 3.0, 0.0, -0.125, 7.0], dtype=np.float32)
    got = o.project_bias("q4", x, payload, pairs, bias)
    for i in range(4):
        for j in range(6):
            acc = Fraction(0)
            for k in range(64):
                byte = int(payload[j, k // 2])
                code = byte & 15 if k % 2 == 0 else byte >> 4
                acc += int(x[i, k]) * (Fraction(code, 2) - 4)
            assert Fraction(float(got[i, j])) == acc + Fraction(float(bias[j])), (i, j)
    zero = o.project_bias("q4", np.zeros((3, 64), dtype=np.float32), payload, pairs, bias)
    assert np.array_equal(zero, np.broadcast_to(bias.astype(np.float64), (3, 6)))


PINS_BIAS = [pin_project_bias]


def _sqrt_fraction_close(value, square: Fraction, rel=1e-15):
    """value ~ sqrt(square), checked as value**2 against the exact rational square."""
    assert value >= 0.0 and math.isfinite(value), value
    v = Fraction(value)
    assert abs(v * v - square) <= rel * square, (value, float(square))


def pin_rel_fro(o):
    """The parity metric ||y - y_ref||_F / ||y_ref||_F (the 1e-5 bar of the
    fp32-activation GEMM is stated as a relative Frobenius error), checked on
    hand-computed cases whose exact values follow from the definition."""
    # [[4, 4]] against [[3, 4]]: difference (1, 0), reference norm 5 -> 1/5.
    # Normalising by ||y|| would give 1/sqrt(32), the max-abs ratio 1/4, the
    # squared ratio 1/25.
    assert o.rel_fro(np.array([[4.0, 4.0]]), np.array([[3.0, 4.0]])) == 0.2
    # the argument order matters: [[3, 4]] against [[4, 4]] is 1/sqrt(32)
    _sqrt_fraction_close(o.rel_fro(np.array([[3.0, 4.0]]), np.array([[4.0, 4.0]])), Fraction(1, 32))
    # Frobenius over the whole tensor, not the worst row: rows (3, 4) and
    # (6, 8), one unit off in the first row -> 1/sqrt(125) (the worst row
    # alone would give 1/5)
    _sqrt_fraction_close(o.rel_fro(np.array([[3.0, 5.0], [6.0, 8.0]]), np.array([[3.0, 4.0], [6.0, 8.0]])),
                         Fraction(1, 125))
    # not the spectral norm: identity reference, one diagonal entry off by 1
    # -> 1/sqrt(2) (spectral norms would give 1)
    _sqrt_fraction_close(o.rel_fro(np.array([[2.0, 0.0], [0.0, 1.0]]), np.eye(2)), Fraction(1, 2))
    # a 3-D tensor is measured over all of its elements as well
    ref3 = np.zeros((2, 2, 2))
    ref3[0, 0, 0] = 3.0
    ref3[1, 1, 1] = 4.0
    got3 = ref3.copy()
    got3[1, 0, 1] = 1.0
    assert o.rel_fro(got3, ref3) == 0.2
    # equal tensors -> 0; both zero -> 0; a nonzero result against a zero
    # reference -> infinity (no finite relative error exists)
    y = np.arange(12, dtype=np.float32).reshape(3, 4) - 5.5
    assert o.rel_fro(y, y) == 0.0
    assert o.rel_fro(np.zeros((2, 3)), np.zeros((2, 3))) == 0.0
    assert o.rel_fro(np.array([[0.0, 1e-30]]), np.zeros((1, 2))) == float("inf")
    # fp32 inputs are measured in fp64: a difference of one fp32 ulp at 1.0
    # among 10^4 equal entries is 2^-23 / 100 relative, not rounded to zero
    big = np.ones((100, 100), dtype=np.float32)
    one_off = big.copy()
    one_off[7, 9] = np.float32(1.0 + 2.0 ** -23)
    _sqrt_fraction_close(o.rel_fro(one_off, big), Fraction(1, 2 ** 46 * 10 ** 4))
    # scale invariance by a power of two, and a NaN in the result never passes the bar
    yr = np.array([[1.5, -2.0, 0.25]])
    yg = np.array([[1.5, -2.0, 0.5]])
    assert o.rel_fro(yg * 2.0 ** 60, yr * 2.0 ** 60) == o.rel_fro(yg, yr) == o.rel_fro(yg * 2.0 ** -60, yr * 2.0 ** -60)
    assert not (o.rel_fro(np.array([[np.nan, 1.0]]), np.array([[1.0, 1.0]])) <= 1e-5)


PINS_METRIC = [pin_rel_fro]


PINS = [pin_nibble_golden, pin_pack_roundtrip, pin_q4_dequant_golden, pin_q4_dequant_identity_probe,
        pin_q4_dequant_rational, pin_q8_dequant_rational, pin_q8_golden, pin_q8_closed_form,
        pin_q4_recon_bound, pin_q4_grid_roundtrip, pin_q4_clip_argmin, pin_q4_degenerate,
        pin_gemm_triple_loop, pin_gemm_exact_integer] + PINS_F8 + PINS_BF16 + PINS_BIAS + PINS_METRIC


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


# ----------------------------------------------------------------------------
# The library primitives the oracle leans on.
# ----------------------------------------------------------------------------
@pytest.mark.filterwarnings("ignore:overflow encountered")
def test_numpy_f64_to_f16_is_correctly_rounded():
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000))
    ulp1 = 2.0 ** -10
    vals += [1 + ulp1 / 2, 1 + 3 * ulp1 / 2, 1 + ulp1 / 2 + 2 ** -40, 1 + ulp1 / 2 - 2 ** -40,
             2 ** -24, 2 ** -25, 2 ** -25 + 2 ** -60, 3 * 2 ** -25, 65504.0, 65519.99, 65520.0,
             6.0e-5, -2 ** -14 * (1 - 2 ** -11), 0.0]
    for v in vals:
        assert float(np.float64(v).astype(np.float16)) == round_rne(Fraction(v), F16), v


def test_f8_encoder_agrees_with_torch_cast():
    """The oracle's E4M3 encoder (written from the encoding's definition) gives
    the same codes as PyTorch's own cast to float8_e4m3fn, which the FP8 card
    names as the storage type."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    w = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 4, 100000)).astype(np.float32)
    w = np.concatenate([w, np.array([0.0, -0.0, 448, 449, 464, 465, 480, 1e9, np.inf, -np.inf, np.nan,
                                     2 ** -9, 2 ** -10, 3 * 2 ** -11, 2 ** -149], dtype=np.float32)])
    ref = torch.from_numpy(w).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quantize_f8(w), ref)


def test_numpy_fp32_matmul_meets_tolerance():
    """fp32 arithmetic reaches the 1e-5 relative-Frobenius bar with margin, so the
    bar is a fair test of an fp32 GEMM."""
    for K in (512, 2048):
        x = synth.activation(9, 0, "x_attn", 80, K)
        W = synth.weight(9, 0, 0, "wq", 512, K)
        y32 = x @ W.T
        assert oracle.rel_fro(y32, oracle.gemm_ref(x, W)) < 1e-6


def test_recipe_matches_int4_card():
    # int4 card, "Quantization format": int4 for wq/wk/wv/wg and ffn.w1/w3,
    # int8 for the residual-writing wo and ffn.w2.
    assert {k for k, v in oracle.RECIPE_MIXED.items() if v == "q4"} == {"wq", "wk", "wv", "wg", "w1", "w3"}
    assert {k for k, v in oracle.RECIPE_MIXED.items() if v == "q8"} == {"wo", "w2"}
    assert set(oracle.RECIPE_ALL_Q8.values()) == {"q8"}


def test_byte_accounting():
    """q4 stores 0.5 B payload + 4 B per 32 weights (5 bits/weight); q8 1 B per
    weight + 4 B per row. One RT-J block (mixed recipe) is 3,280,896 bytes."""
    total = 0
    for name in synth.PROJ_ORDER:
        N, K, _ = synth.BLOCK_SHAPES[name]
        W = np.zeros((N, K), dtype=np.float32)
        if oracle.RECIPE_MIXED[name] == "q4":
            p, s = oracle.quantize_q4(W)
        else:
            p, s = oracle.quantize_q8(W)
        total += p.nbytes + s.nbytes
    assert total == 3_280_896


# ----------------------------------------------------------------------------
# Planted mistakes: each broken copy must fail at least one pin.
# ----------------------------------------------------------------------------
def _mut_unpack_swapped(payload):
    q = oracle.unpack_q4(payload)
    return q.reshape(q.shape[0], -1, 2)[:, :, ::-1].reshape(q.shape).copy()


def _mut_dequant_q4_no_min(payload, pairs):
    p = np.array(pairs, dtype=np.float16, copy=True)
    p[..., 1] = 0
    return oracle.dequant_q4(payload, p)


def _mut_dequant_q4_pair_swapped(payload, pairs):
    return oracle.dequant_q4(payload, np.asarray(pairs)[..., ::-1])


def _mut_dequant_q4_group_shift(payload, pairs):
    return oracle.dequant_q4(payload, np.roll(np.asarray(pairs), 1, axis=1))


def _mut_dequant_q4_fp16_rounded(payload, pairs):
    return oracle.dequant_q4(payload, pairs).astype(np.float16).astype(np.float32)


def _mut_dequant_q8_row_shift(q, scale):
    return oracle.dequant_q8(q, np.roll(np.asarray(scale), 1))


def _mut_quantize_q8_div128(W):
    W = np.asarray(W, dtype=np.float32)
    scale = (np.abs(W).max(axis=1).astype(np.float64) / 128.0).astype(np.float32)
    q = np.zeros(W.shape)
    live = scale > 0
    q[live] = np.clip(np.rint(W[live] / scale[live, None].astype(np.float64)), -127, 127)
    return q.astype(np.int8), scale


def _mut_quantize_q8_trunc(W):
    q, scale = oracle.quantize_q8(W)
    W64 = np.asarray(W, dtype=np.float64)
    live = scale > 0
    qt = np.zeros(W64.shape)
    qt[live] = np.clip(np.trunc(W64[live] / scale[live, None]), -127, 127)
    return qt.astype(np.int8), scale


def _mut_quantize_q4_no_search(W, return_alpha=False):
    orig = oracle.rtq_oracle.CLIP_GRID
    try:
        oracle.rtq_oracle.CLIP_GRID = (1.0,)
        return oracle.quantize_q4(W, return_alpha=return_alpha)
    finally:
        oracle.rtq_oracle.CLIP_GRID = orig


def _mut_quantize_q4_midpoint_shrink(W, return_alpha=False):
    orig = oracle.rtq_oracle._q4_candidate

    def cand(w, wmin, wmax, alpha):
        mid = 0.5 * (wmin + wmax)
        return orig(w, mid + alpha * (wmin - mid), mid + alpha * (wmax - mid), 1.0)
    try:
        oracle.rtq_oracle._q4_candidate = cand
        return oracle.quantize_q4(W, return_alpha=return_alpha)
    finally:
        oracle.rtq_oracle._q4_candidate = orig


def _mut_quantize_q4_floor(W, return_alpha=False):
    orig = np.rint
    try:
        oracle.rtq_oracle.np.rint = np.floor
        return oracle.quantize_q4(W, return_alpha=return_alpha)
    finally:
        oracle.rtq_oracle.np.rint = orig


def _mut_gemm_no_transpose(x, W):
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64)


def _mut_gemm_drop_last_k(x, W):
    return np.asarray(x, np.float64)[:, :-1] @ np.asarray(W, np.float64)[:, :-1].T


def _mut_gemm_fp32(x, W):
    return (np.asarray(x, np.float32) @ np.asarray(W, np.float32).T).astype(np.float16).astype(np.float64)


def _mut_project_q4_transposed(x, payload, pairs):
    W = oracle.dequant_q4(payload, pairs)
    return np.asarray(x, np.float64) @ W.astype(np.float64)[:, ::-1].T


def test_bf16_rounding_agrees_with_torch_cast():
    """The oracle's bf16 rounding (written from the format's definition) gives
    the same bits as PyTorch's float32 -> bfloat16 cast."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(23)
    x = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = x[((x >> 23) & 0xFF) != 0xFF].view(np.float32)
    x = np.concatenate([x, (rng.standard_normal(100000)).astype(np.float32),
                        np.array([np.inf, -np.inf, 0.0, -0.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.round_bf16(x).view(np.uint32), ref.view(np.uint32))


def _mut_round_bf16_truncate(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32)


def _mut_round_bf16_ties_away(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return (((b + 0x8000) & 0xFFFF0000).astype(np.uint32)).view(np.float32)


def _mut_project_bf16_unrounded(fmt, x, payload, scale):
    return oracle.project(fmt, x, payload, scale)


def _mut_project_bias_rows(fmt, x, payload, scale, bias):
    y = oracle.project(fmt, x, payload, scale)
    b = np.asarray(bias, dtype=np.float64)
    return y + np.resize(b, y.shape[0])[:, None]


def _mut_project_bias_dropped(fmt, x, payload, scale, bias):
    return oracle.project(fmt, x, payload, scale)


def _mut_decode_f8_bias8(codes):
    return oracle.decode_f8(codes) / 2.0


def _mut_decode_f8_no_subnormals(codes):
    v = oracle.decode_f8(codes)
    c = np.asarray(codes, dtype=np.uint8)
    return np.where(((c >> 3) & 0xF) == 0, 0.0, v)


def _mut_quantize_f8_ties_away(W):
    w = np.asarray(W, dtype=np.float32)
    out = oracle.quantize_f8(w)
    # bump every exact midpoint to the larger magnitude
    lo = oracle.decode_f8(out & 0x7F)
    hi = oracle.decode_f8(np.minimum((out & 0x7F) + 1, 0x7E))
    mid = np.abs(w.astype(np.float64)) == (lo + hi) / 2
    return np.where(mid & ((out & 0x7F) < 0x7E), out + 1, out).astype(np.uint8)


def _mut_quantize_f8_saturate(W):
    out = oracle.quantize_f8(W)
    w = np.asarray(W, dtype=np.float32)
    return np.where(((out & 0x7F) == 0x7F) & ~np.isnan(w), (out & 0x80) | 0x7E, out).astype(np.uint8)


def _mut_rel_fro_by_result(y, y_ref):
    y, y_ref = np.asarray(y, np.float64), np.asarray(y_ref, np.float64)
    den = np.linalg.norm(y.ravel())
    return 0.0 if den == 0.0 else float(np.linalg.norm((y - y_ref).ravel()) / den)


def _mut_rel_fro_max_abs(y, y_ref):
    y, y_ref = np.asarray(y, np.float64), np.asarray(y_ref, np.float64)
    den = np.abs(y_ref).max()
    num = np.abs(y - y_ref).max()
    return (0.0 if num == 0.0 else float("inf")) if den == 0.0 else float(num / den)


def _mut_rel_fro_squared(y, y_ref):
    r = oracle.rel_fro(y, y_ref)
    return r * r


def _mut_rel_fro_zero(y, y_ref):
    return 0.0


def _mut_rel_fro_swapped(y, y_ref):
    return oracle.rel_fro(y_ref, y)


def _mut_rel_fro_worst_row(y, y_ref):
    y, y_ref = np.atleast_2d(np.asarray(y, np.float64)), np.atleast_2d(np.asarray(y_ref, np.float64))
    return max(oracle.rel_fro(a, b) for a, b in zip(y, y_ref))


def _mut_rel_fro_spectral(y, y_ref):
    y, y_ref = np.asarray(y, np.float64), np.asarray(y_ref, np.float64)
    if y.ndim != 2:
        return oracle.rel_fro(y, y_ref)
    den = np.linalg.norm(y_ref, 2)
    num = np.linalg.norm(y - y_ref, 2)
    return (0.0 if num == 0.0 else float("inf")) if den == 0.0 else float(num / den)


def _mut_rel_fro_fp32(y, y_ref):
    y, y_ref = np.asarray(y, np.float32), np.asarray(y_ref, np.float32)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    return (0.0 if num == 0.0 else float("inf")) if den == 0.0 else float(np.float32(num) / np.float32(den))


def _mut_rel_fro_zero_ref_passes(y, y_ref):
    y_ref = np.asarray(y_ref, np.float64)
    return 0.0 if np.linalg.norm(y_ref) == 0.0 else oracle.rel_fro(y, y_ref)


MUTANTS = {
    "project_bias_rows": {"project_bias": _mut_project_bias_rows},
    "project_bias_dropped": {"project_bias": _mut_project_bias_dropped},
    "round_bf16_truncate": {"round_bf16": _mut_round_bf16_truncate},
    "round_bf16_ties_away": {"round_bf16": _mut_round_bf16_ties_away},
    "project_bf16_unrounded": {"project_bf16": _mut_project_bf16_unrounded},
    "decode_f8_bias8": {"decode_f8": _mut_decode_f8_bias8},
    "decode_f8_no_subnormals": {"decode_f8": _mut_decode_f8_no_subnormals},
    "quantize_f8_ties_away": {"quantize_f8": _mut_quantize_f8_ties_away},
    "quantize_f8_saturate": {"quantize_f8": _mut_quantize_f8_saturate},
    "unpack_swapped": {"unpack_q4": _mut_unpack_swapped},
    "dequant_q4_no_min": {"dequant_q4": _mut_dequant_q4_no_min},
    "dequant_q4_pair_swapped": {"dequant_q4": _mut_dequant_q4_pair_swapped},
    "dequant_q4_group_shift": {"dequant_q4": _mut_dequant_q4_group_shift},
    "dequant_q4_fp16_rounded": {"dequant_q4": _mut_dequant_q4_fp16_rounded},
    "dequant_q8_row_shift": {"dequant_q8": _mut_dequant_q8_row_shift},
    "quantize_q8_div128": {"quantize_q8": _mut_quantize_q8_div128},
    "quantize_q8_trunc": {"quantize_q8": _mut_quantize_q8_trunc},
    "quantize_q4_no_search": {"quantize_q4": _mut_quantize_q4_no_search},
    "quantize_q4_midpoint_shrink": {"quantize_q4": _mut_quantize_q4_midpoint_shrink},
    "quantize_q4_floor": {"quantize_q4": _mut_quantize_q4_floor},
    "gemm_no_transpose": {"gemm_ref": _mut_gemm_no_transpose},
    "gemm_drop_last_k": {"gemm_ref": _mut_gemm_drop_last_k},
    "gemm_low_precision": {"gemm_ref": _mut_gemm_fp32},
    "project_q4_transposed": {"project_q4": _mut_project_q4_transposed},
    "rel_fro_by_result": {"rel_fro": _mut_rel_fro_by_result},
    "rel_fro_max_abs": {"rel_fro": _mut_rel_fro_max_abs},
    "rel_fro_squared": {"rel_fro": _mut_rel_fro_squared},
    "rel_fro_zero": {"rel_fro": _mut_rel_fro_zero},
    "rel_fro_swapped": {"rel_fro": _mut_rel_fro_swapped},
    "rel_fro_worst_row": {"rel_fro": _mut_rel_fro_worst_row},
    "rel_fro_spectral": {"rel_fro": _mut_rel_fro_spectral},
    "rel_fro_fp32": {"rel_fro": _mut_rel_fro_fp32},
    "rel_fro_zero_ref_passes": {"rel_fro": _mut_rel_fro_zero_ref_passes},
}


def _namespace(overrides):
    mod = oracle.rtq_oracle
    ns = types.SimpleNamespace(**{k: getattr(mod, k) for k in dir(mod) if not k.startswith("__")})
    for k, v in overrides.items():
        setattr(ns, k, v)
    return ns


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    ns = _namespace(MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin(ns)
        except Exception:                                      # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
