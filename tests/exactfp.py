"""Exact rational model of binary32 / bf16 rounding, for pinning the oracle.

Every value is a ``fractions.Fraction``; rounding to a binary format is done
from its definition (nearest representable value, ties to the one with an
even last significand bit).  Nothing here calls the oracle or the HIP path.
"""
from fractions import Fraction
import struct


def _round_binary(x: Fraction, frac_bits: int, emin: int, emax: int) -> Fraction:
    """Round x to the binary format with `frac_bits` stored fraction bits,
    minimum normal exponent emin and maximum exponent emax (nearest, ties to
    even).  Returns +-inf as a float when the result overflows."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                      # subnormals share emin's spacing
    ulp = Fraction(2) ** (e - frac_bits)
    n = a / ulp
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    if r >= Fraction(2) ** (emax + 1):
        return float("inf") * sign
    return sign * r


def f32(x: Fraction) -> Fraction:
    """Round to IEEE binary32."""
    return _round_binary(Fraction(x), 23, -126, 127)


def bf16(x: Fraction) -> Fraction:
    """Round to bfloat16 (8-bit exponent, 7 stored fraction bits)."""
    return _round_binary(Fraction(x), 7, -126, 127)


def f16(x: Fraction) -> Fraction:
    """Round to IEEE binary16 (5-bit exponent, 10 stored fraction bits)."""
    return _round_binary(Fraction(x), 10, -14, 15)


def f16_bits(v) -> int:
    """binary16 bit pattern of a value that is exactly an fp16 (or +-inf)."""
    return struct.unpack("<H", struct.pack("<e", float(v)))[0]


def f32_bits(v) -> int:
    """binary32 bit pattern of a Fraction/float that is exactly a float32."""
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def bf16_bits(v) -> int:
    """bf16 bit pattern of a value that is exactly a bf16 (or +-inf)."""
    return f32_bits(v) >> 16


def rint_half_even(x: Fraction) -> int:
    """Nearest integer, ties to even."""
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl
