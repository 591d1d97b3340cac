"""The layer under HIP graph capture, as the benchmark times it: every
replay of a captured forward equals the eager forward bit for bit, with
eager work and synchronisations between replays, and after new activations
and routing are copied into the captured input buffers (a captured graph
reads its inputs at replay time; nothing in the library may keep state from
the capture)."""
import dataclasses

import pytest
import torch

import moe_inputs
from moe_inputs import Workload
from nvfp4_block_scaled_03_amd import ops
from oracle import routing as oroute

from parity import device, to_np

pytestmark = pytest.mark.gpu

# a decode-sized layer (one-launch front end) and a larger batch (three
# launches), both with the shared expert
SHAPES = [Workload("graph_decode", 64, 256, 128, 32, 4, 1, 0.0, 0.02, 0.01, 1081),
          Workload("graph_big", 1100, 256, 128, 16, 2, 1, 0.0, 0.02, 0.01, 1082)]


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(w, dev, seed):
    v = dataclasses.replace(w, seed=seed)
    x = moe_inputs.activations(v, device=dev)
    ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(v, device=dev)), w.topk)
    return x, torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev)


@pytest.mark.parametrize("variant", ["w4a4", "w4a16", "mxfp4"])
@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_graph_replays_equal_eager(dev, w, variant):
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    w13 = moe_inputs.expert_weights(w, 13, device=dev)
    w2 = moe_inputs.expert_weights(w, 2, device=dev)
    if variant == "mxfp4":
        layer = ops.MxMoELayer(d, ops.quantize_mx_expert_weights(d, w13, w2), device=dev)
        fwd = lambda x, ids, tw, out: layer.forward(x, ids, tw, out=out)
    else:
        layer = ops.MoELayer(d, ops.quantize_expert_weights(d, w13, w2, keep_canonical=False),
                             torch.tensor([0.003], device=dev), device=dev)
        fwd = lambda x, ids, tw, out: layer.forward(x, ids, tw, variant, out=out)
    # static buffers the graph reads and writes
    x, ids, tw = _inputs(w, dev, w.seed)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    fwd(x, ids, tw, out)
    torch.cuda.synchronize()
    eager = out.clone()
    # a second input set, its eager result through separate buffers
    x2, ids2, tw2 = _inputs(w, dev, w.seed + 1)
    out2 = torch.empty_like(out)
    fwd(x2, ids2, tw2, out2)
    torch.cuda.synchronize()
    eager2 = out2.clone()
    assert not torch.equal(eager, eager2)

    for _ in range(2):
        fwd(x, ids, tw, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x, ids, tw, out)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager forward"
        fwd(x2, ids2, tw2, out2)   # eager work on the same layer between replays
        torch.cuda.synchronize()
        assert torch.equal(out2, eager2)
    # new inputs in the captured buffers
    x.copy_(x2)
    ids.copy_(ids2)
    tw.copy_(tw2)
    for r in range(2):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager2), f"replay {r} with new inputs differs"
