"""Exact rounding of rationals to IEEE binary formats, for pinning the
oracle's rounding rules.  Textbook round-to-nearest, ties to even, on
``fractions.Fraction`` values; shares nothing with the oracle."""

from __future__ import annotations

from fractions import Fraction

#: (significand bits including the hidden one, smallest normal exponent)
FP32 = (24, -126)
FP16 = (11, -14)


def _floor_log2(x: Fraction) -> int:
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def round_rne(x: Fraction, fmt) -> Fraction:
    """x rounded to the nearest value of the binary format, ties to the even
    significand (subnormals included; no overflow handling)."""
    p, emin = fmt
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = max(_floor_log2(x), emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = x / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def round_half_even_int(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl
