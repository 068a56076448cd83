"""Exact IEEE binary32 arithmetic on rationals, for pins of the oracle.

Every operation is computed exactly with ``fractions.Fraction`` and then
rounded once to the nearest binary32 value, ties to the even significand
(IEEE 754 roundTiesToEven, subnormals kept, overflow to infinity).  Values
are passed around as binary32 bit patterns (Python ints) so that a result can
be compared with the oracle's output bit for bit.

This module shares nothing with the oracle: it knows IEEE 754, not the step.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

_TWO = Fraction(2)
_HALF = Fraction(1, 2)
INF_BITS = 0x7F800000


def decode(bits: int) -> Fraction:
    """Exact value of a finite binary32 bit pattern."""
    bits &= 0xFFFFFFFF
    sign, exp, frac = bits >> 31, (bits >> 23) & 0xFF, bits & 0x7FFFFF
    if exp == 0xFF:
        raise ValueError(f"not finite: {bits:#010x}")
    if exp == 0:
        val = Fraction(frac, 1 << 149)                      # frac * 2^-149
    else:
        val = Fraction((1 << 23) | frac) * _TWO ** (exp - 150)  # 1.frac * 2^(exp-127)
    return -val if sign else val


def encode(q: Fraction) -> int:
    """Nearest binary32 to the rational q, ties to even; +0 for q == 0."""
    if q == 0:
        return 0
    sign = 0
    if q < 0:
        sign, q = 1, -q
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if _TWO ** e > q:
        e -= 1                      # now 2^e <= q < 2^(e+1)
    e = max(e, -126)                # below the normal range the spacing is 2^-149
    ulp = _TWO ** (e - 23)
    n = q / ulp
    whole = n.numerator // n.denominator
    rest = n - whole
    if rest > _HALF or (rest == _HALF and whole % 2 == 1):
        whole += 1
    val = whole * ulp
    if val >= _TWO ** 128:
        return (sign << 31) | INF_BITS
    # val has at most 24 significant bits and a binary32 exponent: the double
    # float(val) is exact, and so is its narrowing.
    out = struct.unpack("<I", struct.pack("<f", float(val)))[0]
    return out | (sign << 31)


def encode_float(x: float) -> int:
    """Nearest binary32 to a Python float (a double, converted exactly)."""
    return encode(Fraction(x))


def from_decimal(s: str) -> int:
    """binary32 nearest to a decimal literal (what `0.95f32` means)."""
    return encode(Fraction(s))


def add(a: int, b: int) -> int:
    return encode(decode(a) + decode(b))


def sub(a: int, b: int) -> int:
    return encode(decode(a) - decode(b))


def mul(a: int, b: int) -> int:
    return encode(decode(a) * decode(b))


def div(a: int, b: int) -> int:
    return encode(decode(a) / decode(b))


def sqrt(a: int) -> int:
    """Correctly rounded square root of a non-negative binary32."""
    q = decode(a)
    if q < 0:
        raise ValueError("sqrt of a negative value")
    if q == 0:
        return a
    K = 200                          # q * 4^K is an integer for every binary32 q
    scaled = q * (1 << (2 * K))
    assert scaled.denominator == 1
    r = math.isqrt(scaled.numerator)
    approx = Fraction(r, 1 << K)
    if r * r != scaled.numerator:
        # the root lies strictly inside (r, r + 1) / 2^K; every rounding
        # boundary is a multiple of 2^-K, so a point inside decides alike
        approx += Fraction(1, 1 << (K + 1))
    return encode(approx)


def bits_of(x: float) -> int:
    """Bit pattern of a Python float rounded to binary32 by numpy's cast."""
    import numpy as np
    return int(np.array([x], np.float32).view(np.uint32)[0])


def value_of(bits: int) -> float:
    """The binary32 pattern as a Python float (exact)."""
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
