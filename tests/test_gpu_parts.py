"""The grouped GEMMs in two parts (short experts, tall experts) on two
streams: for a layer that runs its GEMMs in two parts, the forward with the
tall experts' part on a second stream equals the one-stream forward bit for
bit, eagerly and on every replay of a captured graph (the fork and the join
are part of the graph); and where the GEMMs do not split, part 2 launches
nothing and part 1 is the whole GEMM."""
import ctypes
import dataclasses

import pytest
import torch

import moe_inputs
from moe_inputs import Workload
from nvfp4_block_scaled_03_amd import _lib, ops
from oracle import routing as oroute

from parity import device, to_np

pytestmark = pytest.mark.gpu

# 8 routed rows per expert on average, plus a shared expert holding all 256
# tokens: the short experts stream, the shared one takes 128-row tiles
SPLIT = Workload("parts_split", 256, 512, 256, 128, 4, 1, 0.0, 0.02, 0.01, 1091)


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(w, dev, seed):
    v = dataclasses.replace(w, seed=seed)
    x = moe_inputs.activations(v, device=dev)
    ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(v, device=dev)), w.topk)
    return x, torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev)


def _layer(w, d, variant, dev, side, decoded_copies=None):
    w13 = moe_inputs.expert_weights(w, 13, device=dev)
    w2 = moe_inputs.expert_weights(w, 2, device=dev)
    if variant == "mxfp4":
        layer = ops.MxMoELayer(d, ops.quantize_mx_expert_weights(d, w13, w2), device=dev, side_stream=side)
        return layer, (lambda x, ids, tw, out: layer.forward(x, ids, tw, out=out))
    layer = ops.MoELayer(d, ops.quantize_expert_weights(d, w13, w2, keep_canonical=False),
                         torch.tensor([0.003], device=dev), device=dev, side_stream=side,
                         decoded_copies=decoded_copies)
    return layer, (lambda x, ids, tw, out: layer.forward(x, ids, tw, variant, out=out))


@pytest.mark.parametrize("variant", ["w4a4", "w4a16", "mxfp4"])
def test_two_streams_equal_one_stream(dev, variant):
    w = SPLIT
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    assert _lib.load().grouped_gemm_runs_in_parts(ctypes.byref(d)) == 1
    print(f"\n  two streams {variant} T={w.T} H={w.H} I={w.I} E={w.E}+{w.shared} k={w.topk}", flush=True)
    one, fwd1 = _layer(w, d, variant, dev, None)
    two, fwd2 = _layer(w, d, variant, dev, torch.cuda.Stream())
    assert two.side is not None
    x, ids, tw = _inputs(w, dev, w.seed)
    ref = torch.empty(w.T, w.H, dtype=torch.float32, device=dev)
    fwd1(x, ids, tw, ref)
    out = torch.full_like(ref, float("nan"))
    fwd2(x, ids, tw, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "two-stream forward differs from the one-stream forward"

    # captured: fork and join inside the graph; eager work between replays
    x2, ids2, tw2 = _inputs(w, dev, w.seed + 1)
    ref2 = torch.empty_like(ref)
    fwd1(x2, ids2, tw2, ref2)
    torch.cuda.synchronize()
    assert not torch.equal(ref, ref2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd2(x, ids, tw, out)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs"
        o2 = torch.empty_like(ref)
        fwd2(x2, ids2, tw2, o2)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref2)
    x.copy_(x2)
    ids.copy_(ids2)
    tw.copy_(tw2)
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2), "replay with new inputs differs"


def test_parts_of_an_unsplit_gemm(dev):
    """W4A4 on the codes (no f16 copies) never splits: part 2 of GEMM1 and
    GEMM2 writes nothing, part 1 writes what the whole call writes, and the
    combine alone (part 3) then gives the whole call's output."""
    w = SPLIT
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    layer, fwd = _layer(w, d, "w4a4", dev, None, decoded_copies=False)
    x, ids, tw = _inputs(w, dev, w.seed)
    ref = torch.empty(w.T, w.H, dtype=torch.float32, device=dev)
    fwd(x, ids, tw, ref)
    torch.cuda.synchronize()
    a2_ref = layer.a2_q.clone()
    wq, s = layer.w, ops._stream()
    r = ctypes.byref(d)

    def gemm1(part):
        ops.call("grouped_gemm1_swiglu_part", r, ops._p(layer.a1_q), ops._p(layer.a1_sf), None,
                 ops._p(layer.g1), ops._p(layer.al.sorted_pair), ops._p(layer.al.offsets),
                 ops._p(layer.al.plan), ops._p(wq.prep13), ops._p(wq.g13), ops._p(layer.g2),
                 ops._p(layer.a2_q), ops._p(layer.a2_sf), None, part, s)

    def gemm2(part, out):
        ops.call("grouped_gemm2_combine_part", r, ops._p(layer.a2_q), ops._p(layer.a2_sf), None,
                 ops._p(layer.g2), ops._p(layer.al.offsets), ops._p(layer.al.inv_pos), ops._p(layer.al.plan),
                 ops._p(tw), ops._p(wq.prep2), ops._p(wq.g2), ops._p(out), ops._dtype_code(out),
                 ops._p(layer.ws), layer.ws.numel() * 4, part, s)

    layer.a2_q.fill_(0xAB)
    gemm1(2)
    torch.cuda.synchronize()
    assert bool((layer.a2_q == 0xAB).all()), "part 2 of an unsplit GEMM1 wrote"
    gemm1(1)
    torch.cuda.synchronize()
    assert torch.equal(layer.a2_q, a2_ref)
    out = torch.full_like(ref, float("nan"))
    layer.ws.fill_(float("nan"))
    gemm2(2, out)
    torch.cuda.synchronize()
    assert bool(torch.isnan(layer.ws).all()) and bool(torch.isnan(out).all()), "part 2 wrote"
    gemm2(1, out)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all()), "part 1 of GEMM2 ran the combine"
    gemm2(3, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
