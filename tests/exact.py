"""Exact rational arithmetic for pinning the oracle (test helper).

Rounding here is done on ``fractions.Fraction`` values with integer
arithmetic, independently of the oracle's binary64 code, so the two can only
agree if both follow IEEE round-to-nearest-even.
"""
from fractions import Fraction

import numpy as np

F32 = (24, -126, 127)    # significant bits, min normal exponent, max exponent
BF16 = (8, -126, 127)


def exact(v) -> Fraction:
    """Exact rational value of a finite float (numpy or Python)."""
    return Fraction(float(v))


def round_to(q: Fraction, fmt) -> float:
    """Round a rational to the nearest value of the binary format, ties to even."""
    p, emin, emax = fmt
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * float(r)


def to_f32(q: Fraction) -> np.float32:
    return np.float32(round_to(q, F32))


def to_bf16_bits(q: Fraction) -> np.uint16:
    f = np.float32(round_to(q, BF16))
    return np.uint16(np.array([f], np.float32).view(np.uint32)[0] >> 16)


def bf16_value(bits) -> Fraction:
    u = np.array([int(bits) << 16], np.uint32).view(np.float32)[0]
    return Fraction(float(u))
