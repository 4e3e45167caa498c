"""Exact rational re-computation of the rounding rules, for pinning the oracle.

Written independently of ``oracle``: values are ``fractions.Fraction`` and every
rounding is done on the exact value, so the float64 shortcuts the oracle takes
(exact products, double-rounding arguments) can be checked against it.
"""
from __future__ import annotations

from fractions import Fraction


def _exponent(a: Fraction) -> int:
    """e with 2**e <= a < 2**(e+1) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_sig(x: Fraction, p: int) -> Fraction:
    """Round to p significant bits, nearest, ties to even (normal range only)."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = _exponent(a)
    scale = Fraction(2) ** (p - 1 - e)
    m = a * scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * Fraction(fl) / scale


def rne_int(x: Fraction) -> int:
    """Round to the nearest integer, ties to even."""
    x = Fraction(x)
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)


def fl32(x) -> Fraction:
    return round_sig(Fraction(x), 24)


def bf16(x) -> Fraction:
    return round_sig(Fraction(x), 8)
