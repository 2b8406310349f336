"""Exact-rational reference arithmetic for pinning the oracle (pure Python).

Independent of NumPy: values are fractions.Fraction, and the IEEE roundings
the method needs are written out from the format definitions (binary32:
24-bit significand, exponent >= -126; binary16: 11-bit significand,
exponent >= -14).  Used on tiny inputs only.
"""
from fractions import Fraction
import math

HALF = Fraction(1, 2)


def _round_binary(r: Fraction, mant_bits: int, emin: int, mode: str) -> Fraction:
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = -r if r < 0 else r
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if mode == "rne":
        if rem > HALF or (rem == HALF and fl % 2 == 1):
            fl += 1
    elif mode == "up":             # toward +infinity (for positive r)
        if rem > 0 and sign > 0:
            fl += 1
    else:
        raise ValueError(mode)
    return sign * fl * ulp


def fl32(r: Fraction) -> Fraction:
    """Nearest binary32 value (ties to even); no overflow handling."""
    return _round_binary(Fraction(r), 24, -126, "rne")


def f16_up(r: Fraction) -> Fraction:
    """Smallest binary16 value >= r (r >= 0, in range)."""
    return _round_binary(Fraction(r), 11, -14, "up")


def rne_int(r: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    return round(Fraction(r))


def frac(x) -> Fraction:
    """Exact value of a Python/NumPy float."""
    return Fraction(float(x))


def is_pow2(x: float) -> bool:
    m, _ = math.frexp(x)
    return x > 0 and m == 0.5
