"""Exact binary32 rounding of rationals, written from the IEEE-754 definition.

The activation quantizer's reading (per-block scale xs = amax / 127 as a
correctly rounded float32, code = round-half-even of the correctly rounded
float32 quotient v / xs) is pinned against these helpers. They use only
integer and `fractions.Fraction` arithmetic, never float division, so they do
not share a rounding path with the oracle or the kernels.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_EMIN = -126        # smallest normal exponent of binary32
_MANT = 23          # stored fraction bits
_MAX_FINITE = Fraction((2 ** 24 - 1) * 2 ** (127 - 23))


def rne_int(r: Fraction) -> int:
    """Nearest integer to r, ties to the even integer."""
    q = r.numerator // r.denominator          # floor
    frac = r - q
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return q


def rne_f32(r: Fraction) -> np.float32:
    """The binary32 value nearest to the rational r (ties to even significand),
    subnormals included; overflow gives an infinity."""
    r = Fraction(r)
    if r == 0:
        return np.float32(0.0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, _EMIN)                          # below 2^-126 the spacing stays 2^-149
    ulp = Fraction(2) ** (e - _MANT)
    val = rne_int(a / ulp) * ulp               # may carry to 2^(e+1): still representable
    if val > _MAX_FINITE:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))       # exact: val has at most 24 significant bits


def f32(bits: int) -> np.float32:
    """The float32 with the given bit pattern."""
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def bits(v) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def act_scale(amax) -> np.float32:
    """xs = amax / 127, correctly rounded to binary32."""
    return rne_f32(Fraction(float(amax)) / 127)


def act_code(v, xs) -> int:
    """clamp(round_half_even(f32(v / xs)), -127, 127) with the quotient rounded once to binary32."""
    q = rne_int(Fraction(float(rne_f32(Fraction(float(v)) / Fraction(float(xs))))))
    return max(-127, min(127, q))


def quantize_block(v):
    """Codes, scale and code sum of one block under the reading, from exact arithmetic."""
    v = np.asarray(v, dtype=np.float32)
    amax = max(abs(float(t)) for t in v)
    if amax == 0.0:
        return [0] * len(v), np.float32(0.0), 0
    xs = act_scale(amax)
    q = [act_code(t, xs) for t in v]
    return q, xs, sum(q)
