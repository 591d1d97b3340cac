"""Pins for the routing, permutation and layer oracle (CPU only)."""
import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import moe_inputs
from oracle import bruteforce, moe, nvfp4, routing


# ---------------------------------------------------------------- routing
def test_route_closed_form_equals_two_step():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((64, 32)).astype(np.float32)
    ids, w = routing.route_topk(z, 6)
    ids2, w2 = routing.route_two_step(z, 6)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w, w2, rtol=1e-6, atol=0)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_route_bruteforce_sort_and_ties():
    z = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5]], dtype=np.float32)
    ids, w = routing.route_topk(z, 4)
    ref = sorted(range(6), key=lambda e: (-float(z[0, e]), e))[:4]
    assert list(ids[0]) == ref == [1, 2, 4, 0]
    assert w[0, 0] == w[0, 1] == w[0, 2]
    rng = np.random.default_rng(4)
    z = rng.integers(-3, 4, (50, 16)).astype(np.float32)    # many ties
    ids, _ = routing.route_topk(z, 5)
    for t in range(50):
        assert list(ids[t]) == sorted(range(16), key=lambda e: (-float(z[t, e]), e))[:5]


def test_route_weights_descending_and_top1():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((20, 10)).astype(np.float32)
    ids, w = routing.route_topk(z, 3)
    assert np.all(np.diff(w, axis=1) <= 0)
    ids1, w1 = routing.route_topk(z, 1)
    assert np.all(w1 == 1.0) and np.array_equal(ids1[:, 0], np.argmax(z, 1))


def test_route_weights_sum_in_expert_order():
    """The FP64 sum of the selected exponentials runs j = 0, 1, ..., k-1 (the
    order the GPU router uses), checked against a plain Python loop."""
    rng = np.random.default_rng(12)
    z = rng.standard_normal((200, 64)).astype(np.float32) * 3
    ids, w = routing.route_topk(z, 10)
    for t in range(200):
        sel = [float(z[t, e]) for e in ids[t]]
        ex = [math.exp(v - sel[0]) for v in sel]
        tot = 0.0
        for v in ex:
            tot += v
        assert [np.float32(v / tot) for v in ex] == list(w[t])


def test_fp32_near_tie_flag_against_fractions():
    """fp32_rounding_near_tie flags exactly the values within rel of a point
    halfway between FP32 neighbours (exact rational distances)."""
    rng = np.random.default_rng(13)
    v = rng.uniform(0.01, 1.0, 3000)
    # values placed at known distances from FP32 midpoints
    f32 = rng.uniform(0.05, 0.9, 300).astype(np.float32).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(f32)[1] - 24)
    mid = f32 + 0.5 * ulp
    rel = 2.0 ** -40
    placed = np.concatenate([mid, mid * (1 + 0.5 * rel), mid * (1 - 0.5 * rel),
                             mid * (1 + 3 * rel), mid * (1 - 3 * rel)])
    v = np.concatenate([v, placed])
    got = routing.fp32_rounding_near_tie(v, rel)
    for x, flag in zip(v, got):
        fx = Fraction(float(x))
        # FP32 neighbours of x by exact search: below = largest FP32 <= x
        lo = Fraction(float(np.float32(x)))
        if lo > fx:
            lo = Fraction(float(np.nextafter(np.float32(x), np.float32(0))))
        hi = Fraction(float(np.nextafter(np.float32(float(lo)), np.float32(2))))
        m = (lo + hi) / 2
        want = abs(fx - m) <= Fraction(rel) * fx
        assert bool(flag) == want, (x, flag)
    assert got[3000:3900].all() and not got[3900:].any()


# ---------------------------------------------------------------- SwiGLU
def _silu_exact(z: float) -> Decimal:
    """silu(z) = z / (1 + e^-z) evaluated with 60 significant decimal digits."""
    with localcontext() as ctx:
        ctx.prec = 60
        dz = Decimal(float(z))
        return dz / (1 + (-dz).exp())


SILU_GRID = np.concatenate([
    np.array([0.0, -0.0, 1e-300, -1e-300, 5e-324, 2.0 ** -30, -2.0 ** -30, 0.5, -0.5, 1.0, -1.0,
              3.0, -3.0, 20.0, -20.0, 36.0, -36.0, 88.0, -88.0, 700.0, -700.0, 709.0, -709.0,
              1e4, 1e300]),
    np.random.default_rng(14).standard_normal(2000) * np.exp(np.random.default_rng(15).uniform(-8, 6, 2000)),
])


def test_silu_against_exact_decimal():
    """moe.silu within 4 ulps of the 60-digit value on a grid that includes
    tiny, huge and large-negative arguments (where exp(-z) is far above 1)."""
    got = moe.silu(SILU_GRID)
    for z, v in zip(SILU_GRID, got):
        ref = float(_silu_exact(z))
        assert math.copysign(1.0, v) == math.copysign(1.0, ref) or ref == 0.0
        assert abs(v - ref) <= 4 * np.spacing(abs(ref)), (z, v, ref)


def test_silu_against_torch():
    """The same grid through torch's FP64 silu (z * sigmoid(z))."""
    ref = torch.nn.functional.silu(torch.from_numpy(SILU_GRID)).numpy()
    assert np.allclose(moe.silu(SILU_GRID), ref, rtol=1e-14, atol=0)
    big = np.array([-745.0, -1000.0, -1e300])      # true values underflow to -0 or a subnormal
    assert np.all(np.abs(moe.silu(big)) <= 1e-320)


def test_swiglu_gate_then_up_against_exact_decimal():
    """h = silu(first half) * second half, element by element at 60 digits;
    swapping the halves or dropping a factor fails."""
    rng = np.random.default_rng(16)
    I = 48
    c = rng.standard_normal((5, 2 * I)) * 4
    h = moe.swiglu(c, I)
    for r in range(5):
        for i in range(I):
            want = _silu_exact(c[r, i]) * Decimal(float(c[r, I + i]))
            assert abs(h[r, i] - float(want)) <= 8 * np.spacing(abs(float(want))) + 1e-300
    swapped = moe.silu(c[:, I:]) * c[:, :I]
    assert not np.allclose(h, swapped)


# ---------------------------------------------------------------- permutation
def _align_brute(ids, E, shared):
    T, k = ids.shape
    pairs = [(int(ids[t, j]), t * k + j) for t in range(T) for j in range(k)]
    if shared:
        pairs += [(E, T * k + t) for t in range(T)]
    slots = E + shared
    rows = []
    for e in range(slots):
        rows += [f for (ex, f) in pairs if ex == e and (ex < E or shared)]
    counts = [sum(1 for (ex, _) in pairs if ex == e) for e in range(slots)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    inv = [-1] * len(pairs)
    for p, f in enumerate(rows):
        inv[f] = p
    return offsets, rows, inv


@pytest.mark.parametrize("E,k,T,shared", [(8, 2, 16, 0), (5, 3, 40, 1), (64, 8, 33, 0), (1, 1, 7, 0)])
def test_align_bruteforce(E, k, T, shared):
    rng = np.random.default_rng(E * 100 + k)
    z = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = routing.route_topk(z, k)
    off, sp, inv = moe.align(ids, E, shared)
    bo, bs, bi = _align_brute(ids, E, shared)
    assert list(off) == bo and list(sp) == bs and list(inv) == bi
    P = T * k + shared * T
    assert off[-1] == P and sorted(sp) == list(range(P))
    assert np.all(inv[sp] == np.arange(P))
    for e in range(E + shared):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)        # ascending f within each expert


def test_align_drops_invalid_ids():
    ids = np.array([[0, 9], [-1, 2], [2, 0]], dtype=np.int32)
    off, sp, inv = moe.align(ids, 4, 0)
    assert list(off) == [0, 2, 2, 4, 4]
    assert list(sp) == [0, 5, 3, 4]
    assert list(inv) == [0, -1, -1, 2, 3, 1]


# ---------------------------------------------------------------- layer
def _tiny_inputs(w, seed_shift=0):
    x = moe_inputs.activations(w).float().numpy()
    z = moe_inputs.router_logits(w).numpy()
    ids, tw = routing.route_topk(z, w.topk)
    w13 = moe_inputs.expert_weights(w, 13).numpy()
    w2 = moe_inputs.expert_weights(w, 2).numpy()
    return x, ids, tw, w13, w2


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
def test_layer_grouped_equals_per_token(variant):
    w = moe_inputs.WORKLOADS["tiny"]
    x, ids, tw, w13, w2 = _tiny_inputs(w)
    ew = moe.ExpertWeights.from_arrays(w13, w2)
    g2 = moe.calibrate_g2(x, ids, ew, w.E, w.I)
    res = moe.layer(x, ids, tw, ew, w.E, w.I, variant=variant, g2=g2)
    w13h = np.stack([ew.dequantized(13, e) for e in range(w.E)])
    w2h = np.stack([ew.dequantized(2, e) for e in range(w.E)])
    ref = bruteforce.layer_per_token(x, ids, tw, w13h, w2h, w.I, variant=variant, g2=g2)
    assert np.allclose(res.out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    rms = np.sqrt((ref ** 2).mean())
    assert rms > 0


def test_layer_shared_expert_equals_per_token():
    w = moe_inputs.Workload("tiny_shared", 12, 128, 64, 6, 3, 1, 1.1, 0.02, 0.01, 77)
    x = moe_inputs.activations(w).float().numpy()
    ids, tw = routing.route_topk(moe_inputs.router_logits(w).numpy(), w.topk)
    w13 = moe_inputs.expert_weights(w, 13).numpy()
    w2 = moe_inputs.expert_weights(w, 2).numpy()
    ew = moe.ExpertWeights.from_arrays(w13, w2)
    g2 = moe.calibrate_g2(x, ids, ew, w.E, w.I, shared=1)
    res = moe.layer(x, ids, tw, ew, w.E, w.I, g2=g2, shared=1)
    w13h = np.stack([ew.dequantized(13, e) for e in range(w.E + 1)])
    w2h = np.stack([ew.dequantized(2, e) for e in range(w.E + 1)])
    ref = bruteforce.layer_per_token(x, ids, tw, w13h[:w.E], w2h[:w.E], w.I, g2=g2,
                                     shared_w13=w13h[w.E], shared_w2=w2h[w.E])
    assert np.allclose(res.out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _dense_mlp(x_hat, W13, W2, I, variant, g2):
    # silu from torch: these special cases must not lean on moe.silu itself
    gate = torch.from_numpy(x_hat @ W13[:I].T)
    h = torch.nn.functional.silu(gate).numpy() * (x_hat @ W13[I:].T)
    if variant == "w4a4":
        h = nvfp4.dequantize(*nvfp4.quantize(h, g2), g2)
    else:
        h = nvfp4.round_to_bf16(h)
    return h @ W2.T


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
def test_single_expert_top1_is_dense_mlp(variant):
    w = moe_inputs.Workload("dense", 24, 128, 64, 1, 1, 0, 0.0, 0.02, 0.01, 31)
    x = moe_inputs.activations(w).float().numpy().astype(np.float64)
    ids = np.zeros((w.T, 1), dtype=np.int32)
    tw = np.ones((w.T, 1), dtype=np.float32)
    ew = moe.ExpertWeights.from_arrays(moe_inputs.expert_weights(w, 13).numpy(),
                                       moe_inputs.expert_weights(w, 2).numpy())
    g2 = np.float32(0.001)
    res = moe.layer(x, ids, tw, ew, 1, w.I, variant=variant, g2=g2)
    if variant == "w4a4":
        g1 = nvfp4.global_scale(x)
        xh = nvfp4.dequantize(*nvfp4.quantize(x, g1), g1)
    else:
        xh = x
    ref = _dense_mlp(xh, ew.dequantized(13, 0), ew.dequantized(2, 0), w.I, variant, g2)
    assert np.allclose(res.out, ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_is_dense_mlp():
    w = moe_inputs.Workload("same", 20, 128, 64, 6, 3, 0, 0.0, 0.02, 0.01, 41)
    x = moe_inputs.activations(w).float().numpy().astype(np.float64)
    ids, tw = routing.route_topk(moe_inputs.router_logits(w).numpy(), 3)
    W13 = moe_inputs.expert_weight(w, 13, 0).numpy()
    W2 = moe_inputs.expert_weight(w, 2, 0).numpy()
    ew = moe.ExpertWeights(lambda e: W13, lambda e: W2)
    g2 = np.float32(0.002)
    res = moe.layer(x, ids, tw, ew, w.E, w.I, g2=g2)
    g1 = nvfp4.global_scale(x)
    xh = nvfp4.dequantize(*nvfp4.quantize(x, g1), g1)
    ref = _dense_mlp(xh, ew.dequantized(13, 0), ew.dequantized(2, 0), w.I, "w4a4", g2)
    # The router weights sum to 1 up to their FP32 rounding.
    assert np.allclose(res.out, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_w4a16_equals_w4a4_gemm1_on_grid_inputs():
    # x already on the NVFP4 grid with a power-of-two global scale: quantising
    # it is the identity, so both variants see the same GEMM1 input and h.
    w = moe_inputs.Workload("grid", 16, 128, 64, 4, 2, 0, 0.0, 0.02, 0.0, 55)
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, (w.T, w.H)).astype(np.uint8)
    codes[:, ::16] = 7                                # block max code 6
    sc = rng.integers(0x30, 0x48, (w.T, w.H // 16)).astype(np.uint8)
    sc[0, 0] = 0x7E                                   # amax = 6 * 448 * g1
    g1 = np.float32(2.0 ** -4)
    x = nvfp4.dequantize(codes, sc, g1)
    assert nvfp4.global_scale(x) == g1
    assert np.array_equal(torch.tensor(x).to(torch.bfloat16).double().numpy(), x)
    ids, tw = routing.route_topk(moe_inputs.router_logits(w).numpy(), 2)
    ew = moe.ExpertWeights.from_arrays(moe_inputs.expert_weights(w, 13).numpy(),
                                       moe_inputs.expert_weights(w, 2).numpy())
    r4 = moe.layer(x, ids, tw, ew, w.E, w.I, variant="w4a4", g2=np.float32(1e-3))
    r16 = moe.layer(x, ids, tw, ew, w.E, w.I, variant="w4a16")
    assert np.array_equal(r4.h, r16.h)


def test_down_and_combine_matches_layer():
    w = moe_inputs.WORKLOADS["tiny"]
    x, ids, tw, w13, w2 = _tiny_inputs(w)
    ew = moe.ExpertWeights.from_arrays(w13, w2)
    g2 = moe.calibrate_g2(x, ids, ew, w.E, w.I)
    res = moe.layer(x, ids, tw, ew, w.E, w.I, g2=g2)
    a2_hat = nvfp4.dequantize(res.a2_codes, res.a2_scales, g2)
    out = moe.down_and_combine(a2_hat, res.rows, res.sorted_pair, res.offsets, tw, ew, w.T, w.topk)
    assert np.allclose(out, res.out, rtol=1e-12, atol=1e-14)


def test_token_subset_matches_full():
    w = moe_inputs.WORKLOADS["tiny"]
    x, ids, tw, w13, w2 = _tiny_inputs(w)
    ew = moe.ExpertWeights.from_arrays(w13, w2)
    g2 = np.float32(0.001)
    full = moe.layer(x, ids, tw, ew, w.E, w.I, g2=g2)
    sub = moe.layer(x, ids, tw, ew, w.E, w.I, g2=g2, tokens=[1, 5, 11])
    # BLAS may block a smaller product differently: equal to FP64 rounding.
    assert np.allclose(sub.out[[1, 5, 11]], full.out[[1, 5, 11]], rtol=1e-12, atol=1e-15)
    assert not sub.out[[0, 2]].any()


def test_pair_token_weight():
    tw = np.array([[0.25, 0.75], [0.5, 0.5]], dtype=np.float32)
    tok, wt = moe.pair_token_weight(np.array([0, 1, 3, 4, 5]), 2, 2, tw)
    assert list(tok) == [0, 0, 1, 0, 1] and list(wt) == [0.25, 0.75, 0.5, 1.0, 1.0]


def test_layer_calibrate_inline_matches_two_pass():
    """layer(calibrate=True) takes g2 = fl32(max |h| / 2688) over the computed
    pairs: the value calibrate_g2 gives, and then the same layer."""
    w = moe_inputs.WORKLOADS["tiny"]
    x, ids, tw, w13, w2 = _tiny_inputs(w)
    ew = moe.ExpertWeights.from_arrays(w13, w2)
    for toks in (None, [0, 3, 9]):
        g2 = moe.calibrate_g2(x, ids, ew, w.E, w.I, tokens=toks)
        a = moe.layer(x, ids, tw, ew, w.E, w.I, g2=g2, tokens=toks)
        b = moe.layer(x, ids, tw, ew, w.E, w.I, calibrate=True, tokens=toks)
        assert b.g2 == g2
        assert np.array_equal(a.out, b.out) and np.array_equal(a.a2_codes, b.a2_codes)
        # g2 is the global scale of h itself
        assert b.g2 == nvfp4.global_scale(b.h)


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
def test_zero_activations_give_zero(variant):
    """All-zero activations: g1 = 0, every code and block scale 0, and (as
    SwiGLU(0) = 0) a zero intermediate and a zero output, whatever g2."""
    w = moe_inputs.Workload("zeros", 12, 128, 64, 6, 2, 1, 0.0, 0.02, 0.01, 45)
    x = np.zeros((w.T, w.H))
    ids, tw = routing.route_topk(moe_inputs.router_logits(w).numpy(), 2)
    ew = moe.ExpertWeights.from_arrays(moe_inputs.expert_weights(w, 13).numpy(),
                                       moe_inputs.expert_weights(w, 2).numpy())
    res = moe.layer(x, ids, tw, ew, w.E, w.I, variant=variant, g2=np.float32(0.003), shared=1)
    if variant == "w4a4":
        assert nvfp4.global_scale(x) == 0.0
        assert not res.a1_codes.any() and not res.a1_scales.any()
    assert not np.asarray(res.out).any()

