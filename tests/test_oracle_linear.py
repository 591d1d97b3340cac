"""Pins of the dense NVFP4 linear oracle (oracle/linear.py), CPU only.

* Inputs built on the NVFP4 grid (every 16-block holds a code of magnitude 6,
  the tensor maximum sits at scale 448) quantise to themselves, so both
  variants must equal the exact product of the raw inputs, computed here in
  rational arithmetic; the shapes are all different, so a transposed operand
  or a wrong contraction index fails.
* An elementwise Python loop over the dequantised operands (tiny case).
* The expert-layer oracle's down projection with one expert, top-1 and weight 1
  is the same linear map.
"""
from fractions import Fraction

import numpy as np

from oracle import linear as olin
from oracle import moe as omoe
from oracle import nvfp4 as onv


def _grid_matrix(rng, rows, K, g0):
    """Values code * s * g0 with every block's largest magnitude 6 and one
    entry 6 * 448 * g0, so quantisation with g = amax / 2688 = g0 is exact."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    codes = mags[rng.integers(0, 8, (rows, K))] * rng.choice([-1.0, 1.0], (rows, K))
    codes.reshape(rows, K // 16, 16)[:, :, 0] = 6.0
    s = onv.E4M3_POS[rng.integers(1, 127, (rows, K // 16))]
    s[0, 0] = 448.0
    return (codes.reshape(rows, K // 16, 16) * s[..., None]).reshape(rows, K) * g0


def _exact_product(x, w):
    X = [[Fraction(float(v)) for v in row] for row in x]
    W = [[Fraction(float(v)) for v in row] for row in w]
    return [[sum(a * b for a, b in zip(xr, wr)) for wr in W] for xr in X]


def test_grid_inputs_give_the_exact_product():
    rng = np.random.default_rng(7)
    M, N, K = 3, 5, 48
    x = _grid_matrix(rng, M, K, 2.0 ** -6)   # bf16-exact (6 significant bits)
    w = _grid_matrix(rng, N, K, 2.0 ** -12)
    wc, ws, gw = olin.quantize_weight(w)
    assert gw == np.float32(2.0 ** -12)
    assert np.array_equal(onv.dequantize(wc, ws, gw), w)
    exact = _exact_product(x, w)
    for y in (olin.linear_w4a4(x, wc, ws, gw), olin.linear_w4a16(x, wc, ws, gw)):
        assert y.shape == (M, N)
        for m in range(M):
            for n in range(N):
                tol = 1e-13 * float(np.abs(x[m]) @ np.abs(w[n]))
                assert abs(y[m, n] - float(exact[m][n])) <= tol, (m, n)


def test_elementwise_loop():
    rng = np.random.default_rng(8)
    M, N, K = 2, 3, 32
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.1 * rng.standard_normal((N, K))).astype(np.float32)
    wc, ws, gw = olin.quantize_weight(w)
    g = onv.global_scale(x)
    xc, xs = onv.quantize(x, g)
    xh, wh = onv.dequantize(xc, xs, g), onv.dequantize(wc, ws, gw)
    y4, y16 = olin.linear_w4a4(x, wc, ws, gw), olin.linear_w4a16(x, wc, ws, gw)
    for m in range(M):
        for n in range(N):
            a = b = 0.0
            for k in range(K):
                a += xh[m, k] * wh[n, k]
                b += float(x[m, k]) * wh[n, k]
            assert abs(y4[m, n] - a) <= 1e-12 * (1 + abs(a))
            assert abs(y16[m, n] - b) <= 1e-12 * (1 + abs(b))


def test_matches_single_expert_down_projection():
    rng = np.random.default_rng(9)
    T, H, I = 6, 32, 48
    x = rng.standard_normal((T, I)).astype(np.float32)
    w2 = (0.05 * rng.standard_normal((1, H, I))).astype(np.float32)
    weights = omoe.ExpertWeights.from_arrays(np.zeros((1, 2 * I, H), np.float32), w2)
    wc, ws, gw = olin.quantize_weight(w2[0])
    g = onv.global_scale(x)
    xh = onv.dequantize(*onv.quantize(x, g), g)
    ids = np.zeros((T, 1), np.int32)
    off, sp, _ = omoe.align(ids, 1)
    y = omoe.down_and_combine(xh, np.arange(T), sp, off, np.ones((T, 1)), weights, T, 1)
    np.testing.assert_allclose(olin.linear_w4a4(x, wc, ws, gw), y, rtol=1e-13, atol=1e-13)
