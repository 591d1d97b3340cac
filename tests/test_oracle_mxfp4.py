"""Pins of the MXFP4 oracle (oracle/mxfp4.py), CPU only: hand-worked blocks,
the exponent rule against brute force over powers of two, exact round trips
of grid inputs, saturation, ties, and the linear map on grid inputs against
an exact rational product."""
from fractions import Fraction

import numpy as np

from oracle import mxfp4 as omx


def test_hand_worked_block():
    x = np.zeros(32)
    x[:8] = [6.0, -3.0, 0.75, 0.25, 1.25, -0.1, 5.0, 7.0]
    # amax 7 -> floor(log2 7) = 2 -> scale 2^0 (byte 127)
    codes, exps = omx.quantize(x[None])
    assert exps[0, 0] == 127
    # 6 -> 7; -3 -> 8|5; 0.75 tie (0.5, 1) -> even code 2 (1.0); 0.25 tie -> 0;
    # 1.25 tie (1, 1.5) -> 2; -0.1 -> -0 (8); 5 tie (4, 6) -> 6 (4.0); 7 -> saturate 7
    assert list(codes[0, :8]) == [7, 13, 2, 0, 2, 8, 6, 7]
    assert list(codes[0, 8:]) == [0] * 24


def test_exponent_rule_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(300):
        blk = rng.standard_normal(32) * 2.0 ** rng.integers(-30, 30)
        amax = float(np.abs(blk).max())
        e = max(k for k in range(-200, 200) if 2.0 ** k <= amax)   # floor(log2 amax) by search
        assert omx.block_exponents(blk[None])[0, 0] == min(max(e - 2 + 127, 0), 254)
    assert omx.block_exponents(np.zeros((1, 32)))[0, 0] == 0


def test_grid_round_trip_and_nearest():
    rng = np.random.default_rng(4)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(100):
        e = int(rng.integers(-20, 20))
        blk = vals[rng.integers(0, 8, 32)] * rng.choice([-1, 1], 32)
        blk[0] = 6.0 if rng.random() < 0.5 else -4.0   # amax in [4, 8) -> scale 2^0
        x = blk * 2.0 ** e
        c, s = omx.quantize(x[None])
        assert np.array_equal(omx.dequantize(c, s)[0], x)
    # nearest: every dequantised value is a closest grid point to x / X
    x = rng.standard_normal((50, 64)) * 3
    c, s = omx.quantize(x)
    d = omx.dequantize(c, s)
    X = np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=-1)
    grid = np.concatenate([-vals[::-1], vals])[None, None, :] * X[..., None]
    best = np.abs(grid - x[..., None]).min(axis=-1)
    assert np.all(np.abs(d - x) <= best + 1e-15)


def test_linear_grid_exact():
    rng = np.random.default_rng(5)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    def grid(rows, K, e):
        m = vals[rng.integers(0, 8, (rows, K))] * rng.choice([-1, 1], (rows, K))
        m[:, ::32] = 6.0
        return m * 2.0 ** e
    x, w = grid(3, 64, -3), grid(5, 64, -7)
    wc, we = omx.quantize(w)
    y = omx.linear(x, wc, we)
    for i in range(3):
        for j in range(5):
            ex = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[i], w[j]))
            assert y[i, j] == float(ex)
