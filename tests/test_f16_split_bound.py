"""The error bound behind the two-limb fp16 arithmetic, checked with numpy's
own fp16 rounding (no GPU, no library code).

Each row is scaled by 2^e, e = 15 - E with max|x| = f * 2^E, f in [0.5, 1);
every scaled value v is split into h = fp16(v) and l = fp16(v - h), both
rounded to nearest. Claims: the scaled maximum lies in [2^14, 2^15); v - h is
exact in fp32; |v - (h + l)| <= 2^-22 |v| + 2^-25 (scaled units); and
integers of magnitude below 2^22 are carried exactly (h holds the top 11
significant bits, l the next 11, both well above the fp16 subnormal range).
"""
import numpy as np
import pytest


def split_rows(x):
    x = np.asarray(x, dtype=np.float32)
    mx = np.max(np.abs(x), axis=1)
    _, E = np.frexp(mx)
    e = (15 - E).astype(np.int64)
    v = np.ldexp(x.astype(np.float64), e[:, None]).astype(np.float32)     # exact power-of-two scaling
    h = v.astype(np.float16)
    r = v - h.astype(np.float32)                                         # fp32 subtraction
    l = r.astype(np.float16)
    return v, h, r, l, e


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_two_limb_error_bound(seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((64, 512)).astype(np.float32)
    x *= (10.0 ** g.integers(-30, 31, size=(64, 1))).astype(np.float32)
    x[3] = 0.0
    x[5] *= 1e-6
    x[5, 7] = 3.0e4
    v, h, r, l, e = split_rows(x)
    live = np.max(np.abs(x), axis=1) > 0
    vmax = np.max(np.abs(v[live]), axis=1)
    assert np.all(vmax >= 2.0 ** 14) and np.all(vmax < 2.0 ** 15)
    assert np.all(np.isfinite(h))
    # v - h is exact: the fp64 difference equals the fp32 one
    assert np.array_equal(r.astype(np.float64), v.astype(np.float64) - h.astype(np.float64))
    err = np.abs(v.astype(np.float64) - (h.astype(np.float64) + l.astype(np.float64)))
    assert np.all(err <= 2.0 ** -22 * np.abs(v.astype(np.float64)) + 2.0 ** -25)
    # the bound is attained to within a factor: the limbs are not exact in general
    assert np.max(err / np.maximum(np.abs(v.astype(np.float64)), 2.0 ** -3)) > 2.0 ** -26


def test_values_of_22_bits_are_exact():
    g = np.random.default_rng(7)
    ints = g.integers(-(2 ** 21), 2 ** 21, size=(8, 256)).astype(np.float32)   # at most 22 significant bits
    ints[:, 0] = 2.0 ** 21 - 1
    v, h, r, l, e = split_rows(ints)
    assert np.array_equal(v.astype(np.float64), h.astype(np.float64) + l.astype(np.float64))
    small = g.integers(-4, 5, size=(8, 256)).astype(np.float32)
    small[:, 0] = 4.0
    v, h, r, l, e = split_rows(small)
    assert np.all(l == 0) and np.array_equal(v, h.astype(np.float32))
    assert np.all(e == 12)                                  # 4 = 0.5 * 2^3: scaled by 2^12 to 16384
