"""GPU parity: router and permutation by expert, bit for bit (gate G1)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs
from nvfp4_block_scaled_03_amd import _lib, ops
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nvfp4 as onv
from oracle import routing as oroute

from parity import device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def check_router_weights(got, z, ids):
    """Router weights bit for bit.  Both sides take the softmax over the
    selected logits in FP64 (the sum in selection order) and round once to
    FP32; only the exp implementations differ, by an FP64 ulp or two, which
    can move the FP32 rounding only where the FP64 quotient lies within
    2^-40 of a point halfway between FP32 neighbours.  Such positions (the
    oracle flags them; expected none) may differ by one FP32 ulp."""
    sel = np.take_along_axis(np.asarray(z, dtype=np.float32).astype(np.float64), ids.astype(np.int64), axis=1)
    w64 = oroute.selected_weights_f64(sel)
    want = w64.astype(np.float32)
    flag = oroute.fp32_rounding_near_tie(w64)
    diff = got != want
    assert not (diff & ~flag).any(), f"router weights differ at {np.argwhere(diff & ~flag)[:5]}"
    ulp = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert (ulp[diff] <= 1).all()
    print(f"router weights: {diff.sum()} of {got.size} differ, {flag.sum()} flagged near ties")


@pytest.mark.parametrize("name", moe_inputs.ORDER)
def test_router(dev, name):
    w = moe_inputs.WORKLOADS[name]
    z = moe_inputs.router_logits(w, device=dev)
    ids, wt = ops.route_topk(z, w.topk)
    rid, rw = oroute.route_topk(to_np(z), w.topk)
    assert np.array_equal(to_np(ids), rid)
    check_router_weights(to_np(wt), to_np(z), rid)


def test_router_ties(dev):
    z = torch.tensor(np.random.default_rng(1).integers(-2, 3, (300, 40)), dtype=torch.float32, device=dev)
    z[0] = 0.0
    z[1, ::2] = -0.0
    ids, wt = ops.route_topk(z, 7)
    rid, rw = oroute.route_topk(to_np(z), 7)
    assert np.array_equal(to_np(ids), rid)
    check_router_weights(to_np(wt), to_np(z), rid)


def _check_align(dev, ids_np, E, shared, al=None):
    T, k = ids_np.shape
    d = ops.dims(T, k, E, 128, 128, shared)
    if al is None:
        al = ops.moe_align(d, torch.from_numpy(ids_np).to(dev))
    off, sp, inv = omoe.align(ids_np, E, shared)
    P = T * k + shared * T
    n_kept = int(off[-1])
    assert np.array_equal(to_np(al.offsets), off)
    assert np.array_equal(to_np(al.sorted_pair)[:n_kept], sp)
    assert np.array_equal(to_np(al.inv_pos)[:P], inv)
    # The tile lists cover every expert's rows in order, for each tile height
    # (lists 0-3), and for the experts with at most / more than 32 rows in
    # 16- / 128-row tiles (lists 4, 5).
    plan = to_np(al.plan).astype(np.int64) & 0xFFFFFFFF
    lists = [(16, None), (32, None), (64, None), (128, None), (16, True), (128, False)]
    for b, (bm, short) in enumerate(lists):
        cnt, lo = plan[b], plan[6 + b]
        want = []
        for e in range(E + shared):
            n_e = int(off[e + 1] - off[e])
            if short is not None and (n_e <= 32) != short:
                continue
            for m in range((n_e + bm - 1) // bm):
                row0 = int(off[e]) + m * bm
                want += [e | (m << 11), row0 | (min(bm, n_e - m * bm) << 24)]
        assert cnt * 2 == len(want) and list(plan[lo:lo + 2 * cnt]) == want, bm
    return al


@pytest.mark.parametrize("name", moe_inputs.ORDER)
def test_align_workloads(dev, name):
    w = moe_inputs.WORKLOADS[name]
    ids, _ = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    _check_align(dev, ids, w.E, w.shared)


# Pair counts across the alignment paths: one workgroup (P <= 4096), chunk
# scans with the per-expert prefixes in registers (up to 64 chunks of 1024
# pairs) and chunk scans in groups (65 and 80 chunks); past one workgroup
# with 1001 and 1024 expert slots (the tile-list writers' four experts per
# thread, up to the last slot).
@pytest.mark.parametrize("T,k,E,shared", [(1, 1, 1, 0), (1023, 1, 4, 0), (128, 3, 3, 1),
                                          (1025, 1, 1000, 0), (5000, 3, 17, 1), (7, 2, 1023, 1),
                                          (8193, 8, 128, 0), (9000, 8, 64, 1), (6000, 2, 1000, 1),
                                          (4500, 1, 1023, 1)])
def test_align_shapes(dev, T, k, E, shared):
    rng = np.random.default_rng(T + k + E)
    z = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oroute.route_topk(z, k)
    _check_align(dev, ids, E, shared)


@pytest.mark.parametrize("case", ["one_expert", "two_hot", "full_slots"])
def test_align_skewed_one_workgroup(dev, case):
    """The one-workgroup alignment (P <= 4096) at its limits: every pair to
    one expert (4096 rows in one segment), two experts sharing all pairs in
    alternation, and 1023 experts + a shared one (1024 slots, P = 4095),
    each against the oracle's stable grouping and the six tile lists."""
    rng = np.random.default_rng(5)
    if case == "one_expert":
        ids = np.zeros((4096, 1), dtype=np.int32)
        E, shared = 3, 0
    elif case == "two_hot":
        ids = np.stack([np.arange(2048) % 2, 1 - np.arange(2048) % 2], axis=1).astype(np.int32)
        E, shared = 64, 0
    else:
        ids = rng.integers(0, 1023, (455, 8)).astype(np.int32)
        ids[:, 0] = 7          # one hot expert next to many cold ones
        E, shared = 1023, 1
    T, k = ids.shape
    assert T * k + shared * T <= 4096
    _check_align(dev, ids, E, shared)


def test_align_drops_invalid_ids(dev):
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 12, (700, 4)).astype(np.int32)
    ids[::7, 1] = -3
    ids[::11, 2] = 12
    ids[5] = 99
    _check_align(dev, ids, 12, 0)
    _check_align(dev, ids, 12, 1)


def test_align_is_deterministic(dev):
    w = moe_inputs.WORKLOADS["skew"]
    ids, _ = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    t = torch.from_numpy(ids).to(dev)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, 0)
    a = ops.moe_align(d, t)
    b = ops.moe_align(d, t)
    assert torch.equal(a.sorted_pair, b.sorted_pair) and torch.equal(a.inv_pos, b.inv_pos)
    pa, pb = to_np(a.plan), to_np(b.plan)
    assert np.array_equal(pa[:12], pb[:12])      # 6 counts, 6 list offsets
    for i in range(6):          # list entries beyond each count are not written
        lo, n = pa[6 + i], pa[i]
        assert np.array_equal(pa[lo:lo + 2 * n], pb[lo:lo + 2 * n])


def test_align_plan_size_matches(dev):
    d = ops.dims(64, 8, 128, 2048, 768, 0)
    lib = _lib.load()
    assert lib.moe_align_plan_size(ctypes.byref(d)) // 4 == ops.alloc_alignment(d, dev).plan.numel()


@pytest.mark.parametrize("name", ["decode", "large_e", "prefill", "skew", "tiny"])
def test_scale_and_align(dev, name):
    """One call = global scale + alignment (one launch when P <= 4096, the two
    launches otherwise): both results bit-exact, the scale workspace left zero."""
    w = moe_inputs.WORKLOADS[name]
    x = moe_inputs.activations(w, device=dev)
    ids, _ = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    for _ in range(2):
        g, al, gs_ws = ops.scale_and_align(d, x, torch.from_numpy(ids).to(dev))
        assert to_np(g)[0] == onv.global_scale(to_np(x).astype(np.float64))
        _check_align(dev, ids, w.E, w.shared, al=al)
        assert not gs_ws.any()


_LIMIT = moe_inputs.Workload("limit", 128, 2048, 256, 64, 6, 1, 1.1, 0.02, 0.01, 41)  # T*H = 2^18


# 10240 tokens: past the 1024 partial maxima of one load trip each (a
# second, partial trip per thread) and past the 64 chunks whose counts the
# scan keeps in registers.
_BIG = moe_inputs.Workload("big", 10240, 2048, 256, 128, 8, 0, 0.0, 0.02, 0.01, 43)
# 1024 tokens: past one workgroup's pairs but below 2^18 blocks, where the
# fused quantisation takes a lane per 8 elements instead of per block.
_MID = moe_inputs.Workload("mid", 1024, 2048, 256, 64, 8, 0, 0.0, 0.02, 0.01, 44)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["decode", "tiny", "limit", "large_e", "mid", "prefill", "skew", "big"])
def test_quantize_and_align(dev, name):
    """One call = global scale + quantisation (+ exact f16 copy) + alignment,
    bit-exact against the oracle: one launch up to T*H = 2^18 and P = 4096
    (decode, tiny, limit); beyond, three launches -- partial maxima beside
    the chunk counts, the scan (which also finishes g), then the scatter
    and tile lists beside the quantisation (large_e: 3 chunks of pairs, mid:
    8, prefill: 32, skew: 64, big: 80).  (Dense use, no ids, takes the
    scale+align launch then the quantisation: test_gpu_linear.)"""
    w = {"limit": _LIMIT, "big": _BIG, "mid": _MID}.get(name) or moe_inputs.WORKLOADS[name]
    x = moe_inputs.activations(w, device=dev)
    ids, _ = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    xf = to_np(x).astype(np.float64)
    g_ref = onv.global_scale(xf)
    codes, scales = onv.quantize(xf, g_ref)
    for _ in range(2):   # the second call must not depend on state the first left
        deq = torch.empty(w.T, w.H, dtype=torch.float16, device=dev)
        g, q, sf, al = ops.quantize_and_align(d, x, torch.from_numpy(ids).to(dev), deq=deq)
        assert to_np(g)[0] == g_ref
        assert np.array_equal(to_np(q), onv.pack_codes(codes))
        assert np.array_equal(to_np(sf), scales)
        assert np.array_equal(to_np(deq).astype(np.float64), onv.dequantize(codes, scales, 1.0))
        _check_align(dev, ids, w.E, w.shared, al=al)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["decode", "tiny", "limit", "large_e", "mid", "prefill", "skew", "big"])
def test_mx_quantize_and_align(dev, name):
    """One call = OCP MXFP4 quantisation + alignment, bit-exact against the
    oracle: one launch up to P = 4096 (decode, tiny, limit, large_e), the
    quantisation beside the pair scatter and tile lists beyond (prefill,
    skew, big); twice, so that the second call cannot lean on the first."""
    w = {"limit": _LIMIT, "big": _BIG, "mid": _MID}.get(name) or moe_inputs.WORKLOADS[name]
    x = moe_inputs.activations(w, device=dev)
    ids, _ = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    codes, exps = omx.quantize(to_np(x).astype(np.float64))
    for _ in range(2):
        q, ex, al = ops.mx_quantize_and_align(d, x, torch.from_numpy(ids).to(dev))
        assert np.array_equal(onv.unpack_codes(to_np(q)), codes)
        assert np.array_equal(to_np(ex), exps)
        _check_align(dev, ids, w.E, w.shared, al=al)


@pytest.mark.parametrize("name", ["decode", "tiny", "limit", "large_e", "skew", "ties"])
def test_route_and_align(dev, name):
    """One call = router + alignment (the 16-lane router for E <= 256, the
    wavefront router for large_e's E = 512).  Ids and alignment bit-exact,
    weights as in the router test."""
    if name == "ties":
        z = torch.tensor(np.random.default_rng(5).integers(-2, 3, (100, 40)), dtype=torch.float32, device=dev)
        T, E, k, shared = 100, 40, 7, 1
    else:
        w = _LIMIT if name == "limit" else moe_inputs.WORKLOADS[name]
        z = moe_inputs.router_logits(w, device=dev)
        T, E, k, shared = w.T, w.E, w.topk, w.shared
    d = ops.dims(T, k, E, 128, 128, shared)
    rid, rw = oroute.route_topk(to_np(z), k)
    for _ in range(2):
        ids, wt, al = ops.route_and_align(d, z)
        assert np.array_equal(to_np(ids), rid)
        check_router_weights(to_np(wt), to_np(z), rid)
        _check_align(dev, rid, E, shared, al=al)
