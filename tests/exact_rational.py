"""Exact rational arithmetic for the oracle's matmul pins.

Values are rebuilt from the bit formulas of the element formats ("Bit
Layout", "The E2M1 element" and "The E8M0 shared scale"; the f8E4M3FN
layout named on the dialect page), independently of the oracle's tables, and
sums are rounded to float32 exactly once, round-to-nearest-even.
"""
from fractions import Fraction

import numpy as np


def value_exact(code: int, byte: int, elem_is_e2m1: bool):
    """Signed value of one element code under one E8M0 scale byte (None for 0xFF)."""
    if byte == 0xFF:
        return None
    if elem_is_e2m1:
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)) if e else Fraction(m, 2)
    else:
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    v = mag * Fraction(2) ** (int(byte) - 127)
    return -v if s else v


def round_f32(q: Fraction) -> np.float32:
    """The float32 nearest to the rational q, ties to an even significand."""
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))           # within one float32 step of the answer
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    cands = [v for v in cands if np.isfinite(v)]
    dist = [abs(Fraction(float(v)) - q) for v in cands]
    best = min(dist)
    ties = [v for v, d in zip(cands, dist) if d == best]
    if len(ties) == 1:
        return ties[0]
    return [v for v in ties if int(np.float32(v).view(np.uint32)) % 2 == 0][0]
