"""Exact-rational rounding helpers for the tests (no codec arithmetic)."""
from fractions import Fraction

import numpy as np


def round_f32(q: Fraction) -> Fraction:
    """Exact rational -> nearest binary32 (ties to even), as a rational."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)  # subnormal spacing 2^-149
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def round_f16_bits(v: Fraction) -> int:
    """Exact rational -> binary16 bits, ties to even, overflow to inf."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    if a >= 65520:
        return sign | 0x7C00
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * ulp
    return sign | int(np.float16(float(val)).view(np.uint16))  # val is exactly representable
