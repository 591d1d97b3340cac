"""grouped_gemm2_combine_noalloc (the allocation-free GEMM2 + combine) against
grouped_gemm2_combine through the C ABI: bit-identical outputs on two calls
in a row, the second with a smaller input, and size rejection past the
static scratch."""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs import Workload
from nvfp4_block_scaled_03_amd import _lib, ops

from parity import device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _layer_inputs(w, dev):
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    x = moe_inputs.activations(w, device=dev)
    ids, tw = ops.route_topk(moe_inputs.router_logits(w, device=dev), w.topk)
    wq = ops.quantize_expert_weights(d, moe_inputs.expert_weights(w, 13, device=dev),
                                     moe_inputs.expert_weights(w, 2, device=dev), keep_canonical=False)
    g2 = ops.calibrate_g2(d, x, ids, wq)
    layer = ops.MoELayer(d, wq, g2, device=dev)
    layer.forward(x, ids, tw, "w4a4")          # fills a2 and the alignment
    return d, tw, wq, g2, layer


def _both(d, tw, wq, g2, layer, dt):
    dev = g2.device
    ref = ops.gemm2_w4a4(d, layer.a2_q, layer.a2_sf, g2, layer.al, tw, wq, out_dtype=dt, a2_deq=layer.a2_deq)
    out = torch.full((d.T, d.H), float("nan"), dtype=dt, device=dev)
    ops.gemm2_w4a4_noalloc(d, layer.a2_q, layer.a2_sf, g2, layer.al, tw, wq, out, a2_deq=layer.a2_deq)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_path_twice_shrinking(dev):
    big = moe_inputs.WORKLOADS["decode"]                                   # P = 512, H = 2048
    small = Workload("small", 24, 2048, 768, 16, 2, 1, 0.0, 0.02, 0.01, 99)  # P = 72, shared expert
    for w in (big, small):
        d, tw, wq, g2, layer = _layer_inputs(w, dev)
        for dt in (torch.float32, torch.bfloat16):
            ref, out = _both(d, tw, wq, g2, layer, dt)
            assert torch.equal(ref, out), f"{w.name} {dt}"
            assert not torch.isnan(out.float()).any()


def test_noalloc_large_e_fits_and_prefill_is_rejected(dev):
    lib = _lib.load()
    cap = lib.grouped_gemm2_combine_noalloc_max_bytes()
    assert cap == 48 << 20
    w = moe_inputs.WORKLOADS["large_e"]                                    # P * H * 4 = 46.1 MB
    assert w.pairs * w.H * 4 <= cap
    d, tw, wq, g2, layer = _layer_inputs(w, dev)
    ref, out = _both(d, tw, wq, g2, layer, torch.bfloat16)
    assert torch.equal(ref, out)
    p = moe_inputs.WORKLOADS["prefill"]                                    # P * H * 4 = 268 MB
    dp = ops.dims(p.T, p.topk, p.E, p.H, p.I, p.shared)
    rc = lib.grouped_gemm2_combine_noalloc(ctypes.byref(dp), *([None] * 10), None, 0, None)
    assert rc == _lib.NVFP4_EWORKSPACE
    msg = _lib.last_error()
    assert msg.startswith("grouped_gemm2_combine_noalloc:") and str(cap) in msg, msg
