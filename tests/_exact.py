"""Exact-arithmetic helpers for pinning the oracle (tests only).

These evaluate IEEE-754 rounding from its definition -- the nearest
representable value, ties to the even significand -- by searching the ordered
bit patterns with exact rationals.  They share nothing with ``oracle.c``,
which rounds by bracketing with wide integers.
"""
from __future__ import annotations

import struct
from fractions import Fraction


def f32_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _round_positive(a: Fraction, value_of, top: int) -> int:
    """Bit pattern (0..top) of the nearest value to a > 0, ties to even.
    ``value_of(bits)`` is monotone increasing on [0, top]; ``top`` is the
    pattern of infinity."""
    lo, hi = 0, top
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if value_of(mid) <= a:
            lo = mid
        else:
            hi = mid
    vlo = value_of(lo)
    if vlo == a:
        return lo
    if hi == top:  # above the largest finite value
        largest = value_of(top - 1)
        spacing = largest - value_of(top - 2)
        return top - 1 if a < largest + spacing / 2 else top
    vhi = value_of(hi)
    d_lo, d_hi = a - vlo, vhi - a
    if d_lo < d_hi:
        return lo
    if d_hi < d_lo:
        return hi
    return lo if lo % 2 == 0 else hi


def round_to_f32(x: Fraction) -> float:
    """Nearest binary32 to the rational x (ties to even)."""
    if x == 0:
        return 0.0
    bits = _round_positive(abs(x), lambda b: Fraction(f32_from_bits(b)), 0x7F800000)
    v = f32_from_bits(bits)
    return -v if x < 0 else v


def bf16_value(bits: int) -> Fraction:
    return Fraction(f32_from_bits((bits & 0xFFFF) << 16))


def round_to_bf16_bits(x: Fraction) -> int:
    """Nearest bf16 to the rational x (ties to even), as a bit pattern."""
    if x == 0:
        return 0
    bits = _round_positive(abs(x), bf16_value, 0x7F80)
    return bits | (0x8000 if x < 0 else 0)


def round_half_even(x: Fraction) -> int:
    return round(x)  # Fraction.__round__ rounds half to even


def bf16_ulp(v: float) -> float:
    """Spacing of bf16 values in the binade of |v| (v != 0, finite)."""
    import math
    m, e = math.frexp(abs(v))  # |v| = m * 2^e, m in [0.5, 1)
    return math.ldexp(1.0, max(e - 8, -133))
