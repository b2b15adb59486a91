"""Exact-rational statements of the per-block quantities, for pinning the
oracle (not the GPU path).  Slow; used on tiny tensors only.

Everything here is real-number arithmetic on Fractions: the quotient y/S is
exact, the E2M1 rounding is the nearest grid value with ties to the even
code, the error is exact.  The oracle instead follows the fp32 operation
sequence, so the two agree on codes except where fp32 rounding of y/S lands
on the other side of a grid midpoint, and agree on SSE to within fp32
rounding.
"""
from fractions import Fraction

import numpy as np

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def e2m1_round_exact(a: Fraction) -> int:
    best, best_d = 0, a
    for m in range(1, 8):
        d = abs(a - GRID[m])
        if d < best_d or (d == best_d and m % 2 == 0):
            best, best_d = m, d
    return best


def e4m3_values():
    out = {}
    for c in range(1, 0x7F):
        e, m = c >> 3, c & 7
        out[c] = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return out


E4M3 = e4m3_values()


def block_sse_exact(y, S: Fraction) -> Fraction:
    sse = Fraction(0)
    for v in y:
        fy = Fraction(float(v))
        if S == 0:
            yh = Fraction(0)
        else:
            m = e2m1_round_exact(abs(fy) / S)
            yh = GRID[m] * S * (1 if fy >= 0 else -1)
        sse += (fy - yh) ** 2
    return sse


def brute_force_exact(y, g: Fraction, fmt_e4m3=True):
    """(code, sse) minimising the exact SSE; ties -> smaller code."""
    cands = range(1, 0x7F) if fmt_e4m3 else range(0, 255)
    best = None
    for c in cands:
        S = (E4M3[c] if fmt_e4m3 else Fraction(2) ** (c - 127)) * g
        sse = block_sse_exact(y, S)
        if best is None or sse < best[1]:
            best = (c, sse)
    return best


def all_sse_exact(y, g: Fraction, fmt_e4m3=True):
    cands = range(1, 0x7F) if fmt_e4m3 else range(0, 255)
    res = {}
    for c in cands:
        S = (E4M3[c] if fmt_e4m3 else Fraction(2) ** (c - 127)) * g
        res[c] = block_sse_exact(y, S)
    return res


def as_f64(x):
    return np.float64(float(x))
