"""Exact-rational IEEE rounding, for pinning the oracle's roundings.

Written from the definition of a binary floating-point format, with Python's
``fractions`` only: a value is rounded to the nearest number with a p-bit
significand and an exponent no smaller than emin (subnormals below that),
ties to the even significand.  Nothing here calls NumPy's or torch's casts,
so a test comparing the oracle's output with these roundings checks the
oracle against the definition, not against itself.
"""

import struct
from fractions import Fraction

# (significand bits incl. the hidden one, minimum normal exponent)
FP32 = (24, -126)
FP16 = (11, -14)
BF16 = (8, -126)


def exact(v):
    """The exact rational value of a float (fp16/fp32/fp64 values are all exact doubles)."""
    return Fraction(float(v))


def rn(v, fmt):
    """Round the rational ``v`` to the format ``fmt`` (ties to even); no
    overflow handling (callers stay far from the largest finite values)."""
    p, emin = fmt
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def ulp(v, fmt):
    """Spacing of the format at the (nonzero) rational ``v``."""
    p, emin = fmt
    a = abs(Fraction(v))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    return Fraction(2) ** (max(e, emin) - p + 1)


def f32_next(v, steps):
    """The fp32 value ``steps`` units in the last place away from the fp32
    value ``v`` (same sign, positive v only), via its bit pattern."""
    (u,) = struct.unpack("<I", struct.pack("<f", float(v)))
    (r,) = struct.unpack("<f", struct.pack("<I", u + steps))
    return r


def f32(v):
    """The fp32 value nearest to the rational ``v`` (ties to even), as a float."""
    return float(rn(Fraction(v), FP32))
