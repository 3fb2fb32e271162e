"""Exact-arithmetic model of IEEE binary32 rounding, for pinning the oracle's
floating-point readings.

Values are Python ``Fraction``s (exact rationals); ``rn32`` rounds one to the
nearest binary32 value, ties to the even significand, straight from the
format's definition (24-bit significand, exponents down to -126, subnormal
quantum 2^-149).  Nothing here calls numpy's or the C library's float
arithmetic, so a value computed with it is an independent check of the
oracle's numpy float32 steps.
"""
from fractions import Fraction

import numpy as np

_MIN_EXP = -126      # smallest normal exponent
_SIG_BITS = 24       # significand bits, hidden bit included


def exponent(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(q: Fraction) -> int:
    """Nearest integer to q, ties to the even one."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _rn(q: Fraction, sig_bits: int) -> Fraction:
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    quantum = Fraction(2) ** (max(exponent(a), _MIN_EXP) - (sig_bits - 1))
    r = round_half_even(a / quantum) * quantum
    assert r < Fraction(2) ** 128, "overflow is outside this model"
    return sign * r


def rn32(q: Fraction) -> Fraction:
    """q rounded to the nearest binary32 value, ties to even (finite range)."""
    return _rn(q, _SIG_BITS)


def rn_bf16(q: Fraction) -> Fraction:
    """q rounded to the nearest bfloat16 value (binary32's exponent range, an
    8-bit significand), ties to even (finite range)."""
    return _rn(q, 8)


def bits_bf16(q: Fraction) -> int:
    """bfloat16 bit pattern of a value that rn_bf16 returned."""
    b = bits32(q)
    assert b & 0xFFFF == 0, "not a bfloat16 value"
    return b >> 16


def exact(x) -> Fraction:
    """The exact value of a float32 / float64 number."""
    return Fraction(float(x))


def bits32(q: Fraction) -> int:
    """binary32 bit pattern of a value that rn32 returned."""
    v = np.float32(float(q))
    assert Fraction(float(v)) == q, "not a binary32 value"
    return int(v.view(np.uint32))


def f32_of_bits(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]
