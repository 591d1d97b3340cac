"""Inputs placed on product ties of the exact rounding decisions (shared by a
CPU pin of the oracle and a GPU parity test; not collected by pytest).

A decision of the block quantisation compares a value a with a real
threshold g * M (g the FP32 global scale, M = 6 * an E4M3 midpoint, or
t * s for an E2M1 boundary t and a scale s).  When the exact product g * M
lies exactly halfway between two neighbouring FP32 numbers, the two floats
around it are the hardest inputs for a comparison done in FP32: both are
strictly on one side, at half an ulp.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from oracle import nvfp4 as onv


def product_tie_g(M: Fraction, rng, exp_range=(-20, 4)):
    """(g, g * M): an FP32 g for which the exact product g * M needs 25
    significant bits with the last one set, found by search over random
    mantissas."""
    num = M.numerator
    while True:
        mant = int(rng.integers(1 << 23, 1 << 24))
        P = mant * num
        L = P.bit_length()
        if L > 24 and P % (1 << (L - 24)) == 1 << (L - 25):
            e = int(rng.integers(*exp_range))
            g = Fraction(mant) * Fraction(2) ** (e - 23)
            assert Fraction(float(np.float32(float(g)))) == g
            return float(g), g * M


def float_neighbours(v: Fraction):
    """The FP32 numbers just below and just above the real number v."""
    f = np.float32(float(v))
    lo = f if Fraction(float(f)) < v else np.nextafter(f, np.float32(0))
    return [float(lo), float(np.nextafter(lo, np.float32(np.inf)))]


def product_tie_blocks(rng):
    """(x float64 [n, 16] of FP32 values, g list [n]): blocks whose amax sits
    next to a product-tie scale threshold (every E4M3 midpoint), and blocks
    with elements next to product-tie code thresholds (every E2M1 boundary,
    a spread of scales)."""
    e4 = [Fraction(float(v)) for v in onv.E4M3_POS]
    e2 = [Fraction(float(v)) for v in onv.E2M1_MAGS]
    rows, grow = [], []
    for c in range(1, len(e4) - 1):
        M = 3 * (e4[c] + e4[c + 1])                       # 6 * midpoint
        if M.numerator & (M.numerator - 1) == 0:
            continue                                      # a power of two: no product tie exists
        for _ in range(2):
            g, gM = product_tie_g(M, rng)
            for a in float_neighbours(gM):
                blk = np.float32(rng.uniform(-1, 1, 16) * a * 0.9).astype(np.float64)
                blk[0] = a
                rows.append(blk)
                grow.append(g)
    for c in range(8, 0x70, 3):
        s = e4[c]
        for ti in range(7):
            T = (e2[ti] + e2[ti + 1]) / 2 * s
            if T.numerator & (T.numerator - 1) == 0:
                continue
            g, gT = product_tie_g(T, rng)
            amax = float(np.float32(float(6 * s) * g))   # selects scale s
            blk = np.float32(rng.uniform(-1, 1, 16) * amax).astype(np.float64)
            blk[0] = amax
            xs = float_neighbours(gT)
            blk[1:3] = xs
            blk[3:5] = [-v for v in xs]
            rows.append(blk)
            grow.append(g)
    x = np.array(rows)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    return x, grow
