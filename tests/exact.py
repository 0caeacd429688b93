"""Exact rational helpers for pinning the oracle (no numpy rounding involved).

Correct round-to-nearest-even into a binary floating-point format, written
from the IEEE 754 definition on Python Fractions, so the oracle's fp32/fp16
results can be checked against something other than numpy's own casts.
"""
from __future__ import annotations

import math
from fractions import Fraction

# (significand bits incl. hidden bit, minimum normal exponent, maximum exponent)
F32 = (24, -126, 127)
F16 = (11, -14, 15)
BF16 = (8, -126, 127)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix up to 2^e <= a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_rne(fr: Fraction, fmt=F32) -> float:
    """Round a rational to the nearest value of `fmt` (ties to even); returns a
    Python float holding that value (exact, since fp16/fp32 embed in fp64)."""
    bits, emin, emax = fmt
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (bits - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    res = fl * ulp
    max_finite = (Fraction(2) - Fraction(2) ** (1 - bits)) * Fraction(2) ** emax
    if res > max_finite:
        return sign * math.inf
    return sign * float(res)


def rint_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl
