"""Pins of the MXFP4 oracle (oracle/mxfp4.py), CPU only: hand-worked blocks,
the exponent rule against brute force over powers of two, exact round trips
of grid inputs, saturation, ties, and the linear map on grid inputs against
an exact rational product."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mxfp4 as omx
from oracle import nvfp4

mxfp4 = omx


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


# ---------------------------------------------------------------- MXFP4 MoE layer
def _mx_inputs(w):
    import moe_inputs
    from oracle import routing
    x = moe_inputs.activations(w).float().numpy().astype(np.float64)
    ids, tw = routing.route_topk(moe_inputs.router_logits(w).numpy(), w.topk)
    w13 = moe_inputs.expert_weights(w, 13).numpy()
    w2 = moe_inputs.expert_weights(w, 2).numpy()
    return x, ids, tw, w13, w2


@pytest.mark.parametrize("shared", [0, 1])
def test_mx_layer_equals_per_token_loop(shared):
    """The grouped MXFP4 layer equals the token-by-token dense FP64 loop
    (grouping, permutation, combine and the shared expert all checked)."""
    import moe_inputs
    from oracle import bruteforce
    w = moe_inputs.Workload("mx_tiny", 12, 128, 64, 6, 2, shared, 0.0, 0.02, 0.01, 61 + shared)
    x, ids, tw, w13, w2 = _mx_inputs(w)
    ew = mxfp4.MxExpertWeights.from_arrays(w13, w2)
    res = mxfp4.layer(x, ids, tw, ew, w.E, w.I, shared=shared)
    S = w.E + shared
    w13h = np.stack([ew.dequantized(13, e) for e in range(S)])
    w2h = np.stack([ew.dequantized(2, e) for e in range(S)])
    ref = bruteforce.mx_layer_per_token(x, ids, tw, w13h[:w.E], w2h[:w.E], w.I,
                                        shared_w13=w13h[w.E] if shared else None,
                                        shared_w2=w2h[w.E] if shared else None)
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # the staged second half reproduces the layer from its own a2
    a2 = mxfp4.dequantize(res["a2_codes"], res["a2_exps"])
    again = mxfp4.down_and_combine(a2, res["rows"], res["sorted_pair"], res["offsets"], tw, ew, w.T, w.topk)
    assert np.allclose(again, res["out"], rtol=1e-12, atol=1e-14)


def test_mx_single_expert_is_dense_mlp():
    """E = 1, top-1: the MXFP4 dense MLP written out with torch's silu."""
    import moe_inputs
    w = moe_inputs.Workload("mx_dense", 20, 128, 64, 1, 1, 0, 0.0, 0.02, 0.01, 63)
    x, _, _, w13, w2 = _mx_inputs(w)
    ids = np.zeros((w.T, 1), dtype=np.int32)
    tw = np.ones((w.T, 1), dtype=np.float32)
    ew = mxfp4.MxExpertWeights.from_arrays(w13, w2)
    res = mxfp4.layer(x, ids, tw, ew, 1, w.I)
    W13, W2 = ew.dequantized(13, 0), ew.dequantized(2, 0)
    xh = mxfp4.dequantize(*mxfp4.quantize(x))
    gate = torch.nn.functional.silu(torch.from_numpy(xh @ W13[:w.I].T)).numpy()
    h = gate * (xh @ W13[w.I:].T)
    ref = mxfp4.dequantize(*mxfp4.quantize(h)) @ W2.T
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-13)


def _mx_tie_brute(row, rel, abs_tol):
    rel, abs_tol = Fraction(rel), Fraction(abs_tol)
    vals = [Fraction(float(v)) for v in row]
    amax = max(abs(v) for v in vals)
    block = False
    if amax > 0:
        k = 0
        while Fraction(2) ** k > amax:
            k -= 1
        while Fraction(2) ** (k + 1) <= amax:
            k += 1
        block = any(abs(amax - b) <= rel * b + abs_tol for b in (Fraction(2) ** k, Fraction(2) ** (k + 1)))
    X = Fraction(2) ** (int(mxfp4.block_exponents(np.asarray(row)[None, :])[0, 0]) - 127)
    mags = [Fraction(float(v)) for v in nvfp4.E2M1_MAGS]
    mids = [(mags[i] + mags[i + 1]) / 2 * X for i in range(7)]
    elem = [any(abs(abs(v) - b) <= rel * b + abs_tol for b in mids) for v in vals]
    return elem, block


@pytest.mark.parametrize("rel,abs_tol", [(2.0 ** -12, 0.0), (2.0 ** -12, 2.0 ** -16)])
def test_mx_near_tie_mask_against_fractions(rel, abs_tol):
    rng = np.random.default_rng(71)
    rows = list(rng.standard_normal((60, 32)) * np.exp(rng.uniform(-4, 4, (60, 1))))
    for f in (0.0, 0.5, -0.5, 1.5, -1.5, 3.0):       # amax next to a power of two, elements next to midpoints
        for k in (-3, 0, 2):
            r = rng.uniform(-1, 1, 32) * 2.0 ** k * 0.9
            r[0] = 2.0 ** k * (1 + f * rel) + f * abs_tol
            X = 2.0 ** (k - 2)
            r[5] = 2.5 * X * (1 + f * rel) + f * abs_tol
            r[6] = -0.75 * X * (1 - f * rel) - f * abs_tol
            rows.append(r)
    x = np.array(rows)
    ef, bf = mxfp4.near_tie_mask(x, rel, abs_tol)
    for i in range(x.shape[0]):
        elem, block = _mx_tie_brute(x[i], rel, abs_tol)
        assert bool(bf[i, 0]) == block, i
        assert list(ef[i].astype(bool)) == elem, i
