"""Exact rational helpers for the oracle's pins (test code only).

Written independently of the oracle: integer and ``fractions.Fraction``
arithmetic, so that a rounding mistake in the oracle's numpy code cannot
repeat here.
"""
from fractions import Fraction


def round_fraction_to_f32(fr: Fraction) -> Fraction:
    """Nearest binary32 value to a rational (ties to even), exactly."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                       # subnormal spacing below 2^-126
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def rint_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl
