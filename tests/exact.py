"""Exact-rational helpers for brute-force pins of the oracle (tests only).

These round rationals by enumeration / integer arithmetic, a different mechanism
from the oracle's frexp-and-rint rounding, so that a mistake in either shows up.
"""

from fractions import Fraction

import torch


def e4m3_values_torch():
    """All 256 e4m3fn codes decoded by torch's CPU conversion, as Fractions (None for NaN)."""
    vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    out = []
    for v in vals.tolist():
        out.append(None if v != v else Fraction(v))
    return out


_E4M3 = None


def nearest_e4m3_code(x: Fraction, negative: bool = False) -> int:
    """Nearest finite e4m3fn code to x (|x| <= 448) by enumeration; ties go to the even code.

    `negative` gives the sign for x == 0 (a Fraction has no signed zero)."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3_values_torch()
    sign = 0x80 if (x < 0 or (x == 0 and negative)) else 0
    mag = abs(x)
    best = None
    for code in range(0x7F):  # positive finite codes 0x00..0x7E
        d = abs(_E4M3[code] - mag)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | sign


def nearest_binary(x: Fraction, precision: int, emin: int) -> Fraction:
    """Round x to the nearest binary float with `precision` significant bits and smallest
    normal exponent `emin` (subnormals below), ties to even, with no upper limit."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    mag = abs(x)
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    # adjust so that 2**e <= mag < 2**(e+1)
    while Fraction(2) ** e > mag:
        e -= 1
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (precision - 1))
    units = mag / quantum
    lo = units.numerator // units.denominator
    rem = units - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def nearest_f32(x: Fraction) -> Fraction:
    return nearest_binary(x, 24, -126)


def nearest_bf16(x: Fraction) -> Fraction:
    return nearest_binary(x, 8, -126)
