"""Exact-rational model of IEEE 754 binary32 arithmetic, for brute-forcing the
depthwise oracle on tiny inputs.

Each operation is computed exactly with ``fractions.Fraction`` and then
rounded once to the nearest binary32 value, ties to even, with gradual
underflow and overflow to infinity. Signed zeros, infinities and NaN follow
IEEE 754 (round-to-nearest): an exact zero sum is +0 unless both operands are
-0; an exact zero product takes the xor of the signs.

It uses neither numpy's float32 arithmetic nor the C oracle, so agreement is
evidence about both.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

_HALF = Fraction(1, 2)


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def round_f32(q: Fraction) -> float:
    """Nearest binary32 value to a nonzero rational, ties to even."""
    if q == 0:
        raise ValueError("zero has no sign here; handle it in the caller")
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust so that 2**e <= a < 2**(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                    # below 2**-126 the spacing stays 2**-149
    scale = Fraction(2) ** (23 - e)     # one unit in the last place is 2**(e-23)
    m = a * scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > _HALF or (rem == _HALF and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) / scale
    if val >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(val)            # exact: val is a binary32 value


def _special(*vals) -> bool:
    return any(math.isnan(v) or math.isinf(v) for v in vals)


def mul(a: float, b: float) -> float:
    if _special(a, b):
        return a * b                    # IEEE rules for inf / NaN, as in binary64
    exact = Fraction(a) * Fraction(b)
    if exact == 0:
        return math.copysign(0.0, math.copysign(1.0, a) * math.copysign(1.0, b))
    return round_f32(exact)


def add(a: float, b: float) -> float:
    if _special(a, b):
        return a + b
    exact = Fraction(a) + Fraction(b)
    if exact == 0:
        both_neg = math.copysign(1.0, a) < 0 and math.copysign(1.0, b) < 0
        return -0.0 if both_neg else 0.0
    return round_f32(exact)


def fma(a: float, b: float, c: float) -> float:
    """a*b + c with a single rounding."""
    if _special(a, b, c):
        return a * b + c
    prod = Fraction(a) * Fraction(b)
    exact = prod + Fraction(c)
    if exact == 0:
        if prod == 0:
            psign = math.copysign(1.0, a) * math.copysign(1.0, b)
            both_neg = psign < 0 and math.copysign(1.0, c) < 0
            return -0.0 if both_neg else 0.0
        return 0.0
    return round_f32(exact)
