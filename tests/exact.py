"""Exact-arithmetic helpers for the oracle pins (independent of the oracle).

These decide rounding with Python integers and ``fractions.Fraction`` only,
so that a pin built on them cannot share a mistake with the oracle's numpy
bit manipulations.
"""

import math
import struct
from fractions import Fraction


def f32_of_bits(b):
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def bits_of_f32(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def frac_of_bf16(h):
    return Fraction(f32_of_bits((h & 0xFFFF) << 16))




def round_fraction_to_format(v, mant_bits, emin):
    """Nearest value of a binary format to the exact rational v, ties to even.

    The format has ``mant_bits`` significand bits (implicit bit included) and
    minimum normal exponent ``emin`` (subnormals below it).  Overflow is not
    handled (callers stay in range).  Returns a Fraction.
    """
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2**e <= a < 2**(e+1)
    e = math.floor(math.log2(a.numerator)) - math.floor(math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    m = a / ulp
    n = math.floor(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def round_to_f32(v):
    """Exact rational -> nearest fp32 value (ties even), as a Fraction."""
    return round_fraction_to_format(Fraction(v), 24, -126)


def round_to_bf16(v):
    """Exact rational -> nearest bf16 value (ties even), as a Fraction."""
    return round_fraction_to_format(Fraction(v), 8, -126)


def bf16_bits_of_value(v):
    """bf16 bit pattern of a bf16-representable rational (finite)."""
    f = float(v)
    b = bits_of_f32(f)
    assert b & 0xFFFF == 0, "not a bf16 value"
    return b >> 16


def rne_int(v):
    """Nearest integer to an exact rational, ties to even."""
    n = math.floor(v)
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n
