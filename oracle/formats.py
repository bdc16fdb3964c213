"""Number formats used by the method: FP8 E4M3FN and bfloat16 rounding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name "FP8 PV" (diffusers issue #15014, problem statement) without a
variant. The variant taken is OCP E4M3FN, the FP8 format whose largest finite
value is 448 (the fixed P scale): sign-magnitude, 4 exponent bits with bias 7,
3 mantissa bits, subnormals with step 2^-9, no infinities, and the single NaN
mantissa/exponent pattern S.1111.111. Conversion rounds to nearest, ties to
even, on that value grid, and magnitudes beyond the largest finite value
saturate to 448 (OCP "saturating" conversion). The sign of a value that rounds
to zero is kept (-0 is code 0x80).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_EXP = -6  # exponent of the smallest normal, 2^-6
_E4M3_MANT_BITS = 3

_BF16_MIN_EXP = -126
_BF16_MANT_BITS = 7


def f32(x) -> np.ndarray:
    """Round to IEEE binary32, nearest-even (one rounding from float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _round_to_grid(a: np.ndarray, min_exp: int, mant_bits: int) -> np.ndarray:
    """Round non-negative float64 ``a`` to a binary floating-point grid.

    The grid has ``mant_bits`` fraction bits and smallest normal exponent
    ``min_exp`` (subnormals below it keep the spacing 2^(min_exp-mant_bits)).
    Ties go to the even neighbour. Every step is exact in float64: the
    division and multiplication are by powers of two.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                      # a = m * 2^e, m in [0.5, 1)
    expo = np.maximum(e.astype(np.int64) - 1, min_exp)  # floor(log2 a), clamped
    ulp = np.ldexp(1.0, (expo - mant_bits).astype(np.int32))
    n = np.rint(a / ulp)                    # numpy rint: half to even
    return n * ulp


def fp8_e4m3fn_encode(y) -> np.ndarray:
    """Encode real values as OCP E4M3FN codes (uint8), RNE with saturation.

    ``y`` is taken exactly (float32 or float64 input). NaN maps to 0x7F with
    the sign bit of the input.
    """
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.abs(y)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    val = _round_to_grid(a, _E4M3_MIN_EXP, _E4M3_MANT_BITS)
    val = np.minimum(val, E4M3_MAX)         # saturate (also maps +inf to 448)
    # value -> code
    _, e = np.frexp(val)
    expo = e.astype(np.int64) - 1
    is_sub = (val < 2.0 ** _E4M3_MIN_EXP)
    sub_code = np.rint(val / 2.0 ** (_E4M3_MIN_EXP - _E4M3_MANT_BITS))
    safe_expo = np.where(is_sub, 0, expo)
    frac = val / np.ldexp(1.0, safe_expo.astype(np.int32)) - 1.0
    norm_code = ((safe_expo + 7) << 3) + np.rint(frac * 8.0).astype(np.int64)
    code = np.where(is_sub, sub_code.astype(np.int64), norm_code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def fp8_e4m3fn_decode(codes) -> np.ndarray:
    """Decode OCP E4M3FN codes to float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** (_E4M3_MIN_EXP - _E4M3_MANT_BITS)
    norm = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int32))
    val = np.where(e == 0, sub, norm)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def bf16_round_f64(x) -> np.ndarray:
    """Round float64 values once to bfloat16 (nearest-even); return float32.

    The output of the attention forward is bf16 in the input layout; it is
    formed in float64 and rounded once here. Values beyond the bf16 range
    become +-inf (never reached by attention outputs, which are convex
    combinations of V values).
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    val = _round_to_grid(a, _BF16_MIN_EXP, _BF16_MANT_BITS)
    val = np.where(val >= 2.0 ** 128, np.inf, val)
    out = np.where(neg, -val, val)
    return out.astype(np.float32)


def round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Nearest IEEE binary32 value to a rational number (ties to even).

    Exact: the rational is compared against powers of two and divided by the
    ulp of its binade with integer arithmetic; subnormals keep the spacing
    2^-149. Magnitudes beyond the binary32 range are not expected here.
    """
    fr = Fraction(fr)
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    q = n.numerator // n.denominator
    rem = n - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return np.float32(float(sign * q * ulp))
