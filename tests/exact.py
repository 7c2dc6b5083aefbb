"""Exact rational helpers used to pin the oracle (tests only)."""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def _rn_binary(q: Fraction, prec: int, emin: int) -> Fraction:
    """Round a rational to the nearest binary float with `prec` significand bits
    and minimum normal exponent `emin` (ties to even); no overflow handling."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    big_e = max(e, emin) - (prec - 1)
    m = a / (Fraction(2) ** big_e)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * Fraction(2) ** big_e


def rn32(q: Fraction) -> np.float32:
    r = _rn_binary(Fraction(q), 24, -126)
    return np.float32(float(r))  # r is an fp32 value, exactly representable in fp64


def rn64(q: Fraction) -> float:
    return float(_rn_binary(Fraction(q), 53, -1022))


def frac(x) -> Fraction:
    return Fraction(float(x))


def nearest_level_exact(v: Fraction, levels) -> int:
    """argmin |v - L_i| over exact rationals; ties go to the level farther from zero."""
    lv = [frac(l) for l in levels]
    best = None
    for i, l in enumerate(lv):
        d = abs(v - l)
        key = (d, -abs(l))
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]
