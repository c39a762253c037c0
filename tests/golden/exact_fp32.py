"""Exact rational arithmetic for the fp32 golden files (no oracle, no GPU).

Every value here is computed with ``fractions.Fraction`` from the IEEE-754
definitions: a real number is rounded once to the nearest binary32 value
(ties to even), and an integer rounding is round-half-to-even on the exact
rational.  The golden writers in this folder use these helpers, so their
expected values depend on neither side of the parity tests.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def fp32_round(v: Fraction) -> Fraction:
    """The binary32 value nearest to v (ties to even), for |v| in the
    normal range of binary32 or zero."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "outside the normal range of binary32"
    scaled = a / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = round_half_even(scaled)                   # 24-bit significand (2^24 carries)
    return sign * Fraction(m) * Fraction(2) ** (e - 23)


def round_half_even(v: Fraction) -> int:
    """Nearest integer to v, ties to the even neighbour."""
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def to_f32(v: Fraction) -> np.float32:
    """An exactly representable Fraction as np.float32 (asserts exactness)."""
    f = np.float32(float(v))
    assert Fraction(float(f)) == v, "value is not a binary32 number"
    return f


def f32_hex(f) -> str:
    """A binary32 value written exactly, as a hexadecimal float literal."""
    return float(np.float32(f)).hex()


def from_hex(s: str) -> np.float32:
    v = float.fromhex(s)
    f = np.float32(v)
    assert float(f) == v
    return f
