"""Exact-rational helpers for the oracle's pins.

They implement IEEE binary32 rounding (nearest, ties to even) on Python
Fractions from the definition of the format, independently of NumPy, so the
oracle's float32 steps can be checked against exact arithmetic.
"""
from fractions import Fraction
import math


def fl32(v) -> Fraction:
    """Round a rational to the nearest binary32 value (ties to even)."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e - 23, -149)          # 24-bit significand, subnormals at 2^-149
    scaled = a / Fraction(2) ** quantum_exp
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * Fraction(2) ** quantum_exp


def rint_even(v) -> int:
    """Round a rational to the nearest integer, ties to even."""
    v = Fraction(v)
    n = math.floor(v)
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return int(n)


def ulp32(v) -> Fraction:
    """Spacing of binary32 values at |v| (normal range)."""
    a = abs(Fraction(v))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return Fraction(2) ** max(e - 23, -149)
