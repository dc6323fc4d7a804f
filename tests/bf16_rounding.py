"""Exact bf16 rounding for the output-rounding tests (test infrastructure).

bf16 keeps 8 significant bits (1 implicit + 7 stored) and an 8-bit exponent.
The fp32 -> bf16 store rounds to nearest, ties to even (the reading taken for
ruDNN `history_backward`'s final cast of each gradient element).  This module
computes that rounding of an exact rational number with integer arithmetic
only, so the expected bits do not depend on any float conversion routine, and
builds gradient inputs whose sums are exact in fp32 and land on, just above or
just below a bf16 halfway point.
"""
from __future__ import annotations

from fractions import Fraction


def rne_bf16(x: Fraction) -> Fraction:
    """x rounded to the nearest bf16 value, ties to the even significand.
    Normal range only (|x| in [2^-126, 2^127)); 0 stays 0."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    assert -126 <= e < 127, "outside the normal range"
    ulp = Fraction(2) ** (e - 7)
    n = a / ulp  # in [128, 256)
    whole = n.numerator // n.denominator
    rem = n - whole
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * whole * ulp


def bf16_bits(x: Fraction) -> int:
    """The 16-bit pattern of a bf16-representable normal number (or 0)."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    frac = a / Fraction(2) ** e - 1  # in [0, 1), a multiple of 2^-7
    m = frac * 128
    assert m.denominator == 1, "not a bf16 value"
    return sign | ((e + 127) << 7) | int(m)


def halfway_columns(ncols: int):
    """For each of ncols columns, four bf16-exact addends (hi, lo, c, -c) whose
    exact sum hi + lo is a halfway point of bf16 (a tie), a little above or
    below one, or three quarters of an ulp past hi; hi has exponent -3 .. 4 and
    either sign, and its significand walks through odd and even values (one
    column has significand 255/128 and a tie, so its rounding carries into the
    next binade).  Returns a list of (addends, exact sum)."""
    cols = []
    for d in range(ncols):
        e = d % 8 - 3
        sign = -1 if (d // 8) % 2 else 1
        m = (d * 37 + 5) % 128
        kind = (d // 16) % 4
        if d == ncols - 1:
            m, kind = 127, 0
        hi = Fraction(128 + m, 128) * Fraction(2) ** e
        half = Fraction(2) ** (e - 8)  # half an ulp of hi
        lo = {0: half, 1: half + half / 16, 2: half - half / 16, 3: 3 * half / 2}[kind]
        c = Fraction(2) ** (e + 1)
        addends = [sign * hi, sign * lo, c, -c]
        cols.append((addends, sign * (hi + lo)))
    return cols
