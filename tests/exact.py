"""Exact-arithmetic helpers for pinning the oracle (no numpy float arithmetic).

``round_fraction`` rounds an exact rational to the nearest value of a binary
floating-point format with round-half-to-even, from the format's definition
(p significand bits, minimum normal exponent emin, subnormals below it).
"""
from __future__ import annotations

from fractions import Fraction


def round_fraction(x: Fraction, p: int, emin: int) -> Fraction:
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def f32(x) -> Fraction:
    """Nearest IEEE binary32 value (as an exact Fraction)."""
    return round_fraction(Fraction(x), 24, -126)


def f16(x) -> Fraction:
    """Nearest IEEE binary16 value (as an exact Fraction)."""
    return round_fraction(Fraction(x), 11, -14)


def rint_half_even(x: Fraction) -> int:
    x = Fraction(x)
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def sylvester_entry(i: int, j: int) -> int:
    """Entry (i, j) of the natural-order Sylvester Hadamard matrix: (-1)^popcount(i & j)."""
    return -1 if bin(i & j).count("1") % 2 else 1
