"""Exact-arithmetic brute force used to pin the oracle (tests only).

Independent of oracle.c: dot products are exact rationals (fractions.Fraction),
and rounding to bf16 is a nearest-candidate search over neighbouring bf16 bit
patterns, with ties going to the pattern whose last bit is 0.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def bits_to_fraction(b: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    if math.isinf(f) or math.isnan(f):
        raise ValueError("not finite")
    return Fraction(f)


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def nearest_bf16(v: Fraction) -> tuple[int, bool]:
    """(bits, is_tie) of the bf16 nearest to v; ties to an even last bit.

    Candidates are the bf16 patterns adjacent to the truncation of float(v);
    the nearest is chosen with exact rational distances."""
    if v == 0:
        return 0, False
    neg = v < 0
    a = -v if neg else v
    approx = float(a)
    if approx > 3.4e38:
        return (0xFF80 if neg else 0x7F80), False
    base = _f32_bits(approx) >> 16
    cands = []
    for b in range(max(base - 2, 0), min(base + 3, 0x7F80)):
        cands.append((abs(bits_to_fraction(b) - a), b))
    cands.sort()
    (d0, b0), (d1, b1) = cands[0], cands[1]
    tie = d0 == d1
    if tie and (b0 & 1):
        b0 = b1
    # Values beyond the largest finite bf16 by at least half a spacing overflow.
    max_finite = bits_to_fraction(0x7F7F)
    if a - max_finite >= (max_finite - bits_to_fraction(0x7F7E)) / 2 and a > max_finite:
        b0 = 0x7F80
    return (b0 | (0x8000 if neg else 0)), tie


def exact_dot(a_bits, w_bits) -> Fraction:
    return sum((bits_to_fraction(x) * bits_to_fraction(y) for x, y in zip(a_bits, w_bits)),
               Fraction(0))


def tie_distance(v: Fraction) -> Fraction:
    """Distance from v to the nearest bf16 rounding boundary (a midpoint)."""
    if v == 0:
        return Fraction(1)
    a = abs(v)
    approx = float(a)
    base = _f32_bits(approx) >> 16
    best = None
    for b in range(max(base - 2, 0), min(base + 2, 0x7F7F)):
        mid = (bits_to_fraction(b) + bits_to_fraction(b + 1)) / 2
        d = abs(a - mid)
        best = d if best is None or d < best else best
    return best
