"""Guard bands around every buffer the layer writes (overrun detection).

The per-expert row counts of the grouped GEMMs live on the device and are
trusted, as the per-group shapes of the grouped GEMM in vLLM PR #29242 (debug
trace) are; a wrong count or tile bound would write outside a buffer without
any error.  Here every output, intermediate and workspace buffer of a layer
call sits between two 4 KiB bands of a known byte pattern; after the call
both bands must be intact, and the output must equal that of the same layer
run on ordinary allocations (the path is deterministic).
"""
import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs import Workload
from nvfp4_block_scaled_03_amd import ops

from parity import device

pytestmark = pytest.mark.gpu

BAND = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module")
def dev():
    return device()


class Guarded:
    """Buffers carved out of larger allocations with guard bands on both sides."""

    def __init__(self, dev):
        self.dev = dev
        self.items = []

    def make(self, like: torch.Tensor, zero=False) -> torch.Tensor:
        nbytes = like.numel() * like.element_size()
        full = torch.full((2 * BAND + nbytes,), PATTERN, dtype=torch.uint8, device=self.dev)
        inner = full[BAND:BAND + nbytes]
        if zero:
            inner.zero_()
        self.items.append((full, nbytes))
        return inner.view(like.dtype).view(like.shape)

    def check(self, what):
        torch.cuda.synchronize()
        for i, (full, n) in enumerate(self.items):
            lo = full[:BAND].cpu().numpy()
            hi = full[BAND + n:].cpu().numpy()
            assert (lo == PATTERN).all(), f"{what}: buffer {i} written below its start"
            assert (hi == PATTERN).all(), f"{what}: buffer {i} written past its end ({n} bytes)"


def _guard_layer(layer: ops.MoELayer, g: Guarded):
    for name in ("g1", "a1_q", "a1_sf", "a1_deq", "a2_q", "a2_sf", "a2_deq", "a2_bf16", "ws"):
        t = getattr(layer, name)
        if t is not None:
            setattr(layer, name, g.make(t))
    layer.gs_ws = g.make(layer.gs_ws, zero=True)        # must start zeroed
    al = layer.al
    layer.al = ops.Alignment(offsets=g.make(al.offsets), sorted_pair=g.make(al.sorted_pair),
                             inv_pos=g.make(al.inv_pos), plan=g.make(al.plan),
                             workspace=g.make(al.workspace))


CASES = [
    Workload("g16", 40, 256, 256, 8, 2, 0, 0.0, 0.02, 0.01, 21),
    Workload("g128", 600, 256, 384, 4, 2, 1, 0.0, 0.02, 0.01, 22),
    Workload("g_odd", 300, 384, 640, 3, 1, 0, 0.0, 0.02, 0.01, 23),
    Workload("g_split", 200, 256, 128, 40, 2, 1, 1.3, 0.02, 0.01, 24),
    moe_inputs.WORKLOADS["tiny"], moe_inputs.WORKLOADS["decode"], moe_inputs.WORKLOADS["prefill"],
    moe_inputs.WORKLOADS["large_e"], moe_inputs.WORKLOADS["skew"],
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_layer_writes_stay_inside_buffers(dev, w):
    print(f"guards {w.name}", flush=True)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    x = moe_inputs.activations(w, device=dev)
    ids, tw = ops.route_topk(moe_inputs.router_logits(w, device=dev), w.topk)
    wq = ops.quantize_expert_weights(d, moe_inputs.expert_weights(w, 13, device=dev),
                                     moe_inputs.expert_weights(w, 2, device=dev), keep_canonical=False)
    g2 = ops.calibrate_g2(d, x, ids, wq)
    for variant in ("w4a4", "w4a16"):
        decoded_opts = (None, True, False) if variant == "w4a4" else (None,)
        for decoded in decoded_opts:
            ref_layer = ops.MoELayer(d, wq, g2, device=dev, decoded_copies=decoded)
            ref = ref_layer.forward(x, ids, tw, variant, out_dtype=torch.float32).clone()
            g = Guarded(dev)
            layer = ops.MoELayer(d, wq, g2, device=dev, decoded_copies=decoded)
            _guard_layer(layer, g)
            for dt in (torch.float32, torch.bfloat16):
                out = g.make(torch.empty(w.T, w.H, dtype=dt, device=dev))
                layer.forward(x, ids, tw, variant, out=out)
                g.check(f"{w.name} {variant} decoded={decoded} out={dt}")
                want = ref if dt == torch.float32 else ref.to(torch.bfloat16)
                assert torch.equal(out, want), f"{w.name} {variant} decoded={decoded} {dt}"
            del layer, ref_layer
    torch.cuda.empty_cache()


def _guard_mx_layer(layer: ops.MxMoELayer, g: Guarded):
    for name in ("a1_q", "a1_e", "a2_q", "a2_e", "ws"):
        setattr(layer, name, g.make(getattr(layer, name)))
    al = layer.al
    layer.al = ops.Alignment(offsets=g.make(al.offsets), sorted_pair=g.make(al.sorted_pair),
                             inv_pos=g.make(al.inv_pos), plan=g.make(al.plan),
                             workspace=g.make(al.workspace))


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_mx_layer_writes_stay_inside_buffers(dev, w):
    """The OCP MXFP4 layer on the same shapes: every buffer between guard
    bands, and the output equal to that of the same layer on ordinary
    allocations."""
    print(f"mx guards {w.name}", flush=True)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    x = moe_inputs.activations(w, device=dev)
    ids, tw = ops.route_topk(moe_inputs.router_logits(w, device=dev), w.topk)
    wq = ops.quantize_mx_expert_weights(d, moe_inputs.expert_weights(w, 13, device=dev),
                                        moe_inputs.expert_weights(w, 2, device=dev))
    torch.cuda.empty_cache()
    ref = ops.MxMoELayer(d, wq, device=dev).forward(x, ids, tw, out_dtype=torch.float32).clone()
    g = Guarded(dev)
    layer = ops.MxMoELayer(d, wq, device=dev)
    _guard_mx_layer(layer, g)
    for dt in (torch.float32, torch.bfloat16):
        out = g.make(torch.empty(w.T, w.H, dtype=dt, device=dev))
        layer.forward(x, ids, tw, out=out)
        g.check(f"{w.name} mxfp4 out={dt}")
        want = ref if dt == torch.float32 else ref.to(torch.bfloat16)
        assert torch.equal(out, want), f"{w.name} mxfp4 {dt}"
    del layer, wq
    torch.cuda.empty_cache()
