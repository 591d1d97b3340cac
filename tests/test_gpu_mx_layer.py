"""GPU parity of the OCP MXFP4 expert layer (grouped GEMMs on the scaled FP4
matrix instruction) against the MXFP4 oracle (oracle/mxfp4.py): the
activation codes and exponents bit for bit, the requantised intermediate
exact except at oracle-flagged near ties, and the output within the layer
gate of the staged oracle (its down projection of the GPU's own a2)."""
import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs import Workload
from nvfp4_block_scaled_03_amd import ops
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nvfp4 as onv
from oracle import routing as oroute

from parity import check_a2_mx, check_layer_out, device, relf, to_np

pytestmark = pytest.mark.gpu

SMALL = [
    Workload("mx16", 40, 256, 256, 8, 2, 0, 0.0, 0.02, 0.01, 111),
    Workload("mx32", 100, 256, 128, 8, 2, 0, 0.0, 0.02, 0.01, 112),
    Workload("mx64", 200, 512, 256, 6, 2, 0, 0.5, 0.02, 0.01, 113),
    Workload("mx128", 600, 256, 384, 4, 2, 1, 0.0, 0.02, 0.01, 114),
    # odd chunk counts (K = 384, 640) and a GEMM2 width (384) that leaves half
    # of the last 256-column block idle
    Workload("mx128b", 300, 384, 640, 3, 1, 0, 0.0, 0.02, 0.01, 115),
]


@pytest.fixture(scope="module")
def dev():
    return device()


class MxCase:
    def __init__(self, w: Workload, dev, tokens=None, routing=None):
        """``routing``: (ids [T, k] int32, weights [T, k] f32) given directly
        instead of the router's choice on the workload's logits."""
        self.w = w
        self.d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
        self.x = moe_inputs.activations(w, device=dev)
        if routing is None:
            ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
        else:
            ids, tw = routing
        self.ids_np, self.tw_np = ids, tw
        self.ids = torch.from_numpy(ids).to(dev)
        self.tw = torch.from_numpy(tw).to(dev)
        self.w13 = moe_inputs.expert_weights(w, 13, device=dev)
        self.w2 = moe_inputs.expert_weights(w, 2, device=dev)
        self.ew = omx.MxExpertWeights(lambda e: to_np(self.w13[e]), lambda e: to_np(self.w2[e]))
        self.xf = to_np(self.x).astype(np.float64)
        self.tokens = tokens
        print(f"  mx oracle {w.name}", flush=True)
        self.ref = omx.layer(self.xf, ids, tw, self.ew, w.E, w.I, shared=w.shared, tokens=tokens)
        self.wq = ops.quantize_mx_expert_weights(self.d, self.w13, self.w2)


def _judge(case: MxCase, dev):
    w, ref = case.w, case.ref
    layer = ops.MxMoELayer(case.d, case.wq, device=dev)
    out32 = layer.forward(case.x, case.ids, case.tw, out_dtype=torch.float32).clone()
    out16 = layer.forward(case.x, case.ids, case.tw, out_dtype=torch.bfloat16).clone()
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(torch.bfloat16)), "bf16 output != bf16(f32 output)"
    assert np.array_equal(onv.unpack_codes(to_np(layer.a1_q)), ref["a1_codes"])
    assert np.array_equal(to_np(layer.a1_e), ref["a1_exps"])
    rows = ref["rows"]
    chk = check_a2_mx(to_np(layer.a2_q)[rows], to_np(layer.a2_e)[rows], ref["h"], what=f"{w.name} mx")
    exp = ref["out"] if chk.exact else omx.down_and_combine(
        omx.dequantize(chk.codes, chk.scales), rows, ref["sorted_pair"], ref["offsets"], case.tw_np, case.ew,
        w.T, w.topk)
    toks = np.arange(w.T) if case.tokens is None else np.asarray(case.tokens)
    got = to_np(out32).astype(np.float64)[toks]
    rf, ma = check_layer_out(got, exp[toks], f"{w.name} mxfp4")
    e2e = relf(got, ref["out"][toks])
    assert e2e <= 2e-3, f"end-to-end rel-F {e2e:.2e}"
    print(f"{w.name} mxfp4: relF {rf:.2e} maxabs/rms {ma:.2e} (vs own-a2 oracle {e2e:.2e})")
    return layer


@pytest.mark.parametrize("w", SMALL + [moe_inputs.WORKLOADS["tiny"]], ids=lambda w: w.name)
def test_mx_layer_small(dev, w):
    _judge(MxCase(w, dev), dev)


def test_mx_expert_weights_are_the_oracle_codes(dev):
    """The GPU-quantised expert weights, read back through the layer's
    GEMMs, are the oracle's: a one-expert layer whose activations are one-hot
    rows reproduces columns of W13 (checked through h = silu(gate) * up for
    gate = up = the weight values, compared at a2's precision) -- here simply
    the canonical codes of every expert against the oracle's quantisation."""
    w = Workload("mxw", 8, 256, 128, 5, 1, 1, 0.0, 0.02, 0.01, 117)
    S = w.n_experts
    w13 = moe_inputs.expert_weights(w, 13, device=dev)
    q, e = ops.mx_quantize(w13.reshape(S * 2 * w.I, w.H))
    c_ref, e_ref = omx.quantize(to_np(w13).reshape(S * 2 * w.I, w.H))
    assert np.array_equal(onv.unpack_codes(to_np(q)), c_ref) and np.array_equal(to_np(e), e_ref)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "large_e"])
def test_mx_layer_full_size_every_token(dev, name):
    print(f"mx full-size {name}", flush=True)
    case = MxCase(moe_inputs.WORKLOADS[name], dev)
    layer = _judge(case, dev)
    if name == "large_e":
        # as the benchmark runs it: the tall experts' GEMMs on a second
        # stream give the judged one-stream output bit for bit
        two = ops.MxMoELayer(case.d, case.wq, device=dev, side_stream=torch.cuda.Stream())
        assert two.side is not None
        one = layer.forward(case.x, case.ids, case.tw, out_dtype=torch.float32).clone()
        got = two.forward(case.x, case.ids, case.tw, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, one), "two-stream MXFP4 layer differs from the one-stream layer"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill", "skew"])
def test_mx_layer_full_size_hot_expert(dev, name):
    """Sampled tokens end to end, and every a2 row of the hottest and the
    last non-empty expert."""
    print(f"mx full-size {name}", flush=True)
    w = moe_inputs.WORKLOADS[name]
    toks = np.sort(np.random.default_rng(w.seed + 7).choice(w.T, 12, replace=False))
    case = MxCase(w, dev, tokens=toks)
    layer = _judge(case, dev)
    off, sp = case.ref["offsets"], case.ref["sorted_pair"]
    counts = np.diff(off)
    x_hat = omx.dequantize(case.ref["a1_codes"], case.ref["a1_exps"])
    for e in sorted({int(np.argmax(counts)), int(np.nonzero(counts)[0][-1])}):
        rows = np.arange(off[e], off[e + 1])
        tok, _ = omoe.pair_token_weight(sp[rows], w.T, w.topk, case.tw_np)
        h = omoe.swiglu(x_hat[tok] @ case.ew.dequantized(13, e).T, w.I)
        check_a2_mx(to_np(layer.a2_q)[rows], to_np(layer.a2_e)[rows], h, what=f"{name} mx expert rows")


# Routing by expert row counts (top-1, weight 1, the tokens of an expert
# scattered over the batch) at the expert shape (H = 2048, I = 768), so that
# the tall-tile kernel runs its straight-line bodies for K = 2048 (GEMM1) and
# K = 768 (GEMM2).
RAGGED_COUNTS = [1, 16, 17, 32, 33, 64, 65, 128, 129, 0, 200, 255, 256, 257, 300]
SPLIT_COUNTS = [200, 100, 40, 33, 32, 17, 16, 15, 8, 5, 4, 3, 2, 1, 0, 1] + [3] * 24


def _routed(counts, name, seed, dev):
    w = Workload(name, int(sum(counts)), 2048, 768, len(counts), 1, 0, 0.0, 0.02, 0.01, seed)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    ids = ids[np.random.default_rng(seed).permutation(ids.size)].reshape(-1, 1)
    return MxCase(w, dev, routing=(ids, np.ones((w.T, 1), dtype=np.float32)))


@pytest.mark.timeout(600)
def test_mx_layer_ragged_tile_heights(dev):
    """Every token of a layer whose experts end in 128-row tiles of every
    class of active 16-row groups (1, 2, 4, 8 at both ends of each range)
    plus an empty expert: the tall-tile kernel's four instantiations."""
    case = _routed(RAGGED_COUNTS, "mx_ragged", 81, dev)
    assert case.w.pairs / case.w.E > 96
    _judge(case, dev)


@pytest.mark.timeout(600)
def test_mx_layer_split_short_and_tall_experts(dev):
    """Short experts on average (the 16-row kernel) with a few tall ones
    (more than 32 rows: the tall-tile kernel, a second launch)."""
    case = _routed(SPLIT_COUNTS, "mx_split", 82, dev)
    assert case.w.pairs / case.w.E <= 16 and case.w.T > 64
    _judge(case, dev)


@pytest.mark.timeout(600)
def test_mx_layer_max_experts(dev):
    """1023 routed experts and a shared one (1024 slots, the boundary's
    limit): short experts on the 16-row kernel, the shared expert on the
    tall-tile kernel, every token's shared row in the combine."""
    w = Workload("mx_max_experts", 300, 128, 128, 1023, 4, 1, 0.0, 0.02, 0.01, 1012)
    _judge(MxCase(w, dev), dev)


@pytest.mark.parametrize("T,E,k,shared", [(1, 128, 8, 0), (3, 64, 6, 1)], ids=["one_token", "three_tokens"])
def test_mx_layer_few_tokens(dev, T, E, k, shared):
    """Batch-one decode and a three-token batch (single-row tiles)."""
    _judge(MxCase(Workload(f"mx_{T}_tokens", T, 256, 128, E, k, shared, 0.0, 0.02, 0.01, 1030 + T), dev), dev)


@pytest.mark.parametrize("T", [40, 1100], ids=["one_launch_front", "three_launch_front"])
def test_mx_layer_zero_activations(dev, T):
    """All-zero activations: codes and exponent bytes as the oracle encodes
    a zero tensor, and an exactly zero output."""
    w = Workload("mx_zeros", T, 256, 128, 16, 2, 1, 0.0, 0.02, 0.01, 1042)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    wq = ops.quantize_mx_expert_weights(d, moe_inputs.expert_weights(w, 13, device=dev),
                                        moe_inputs.expert_weights(w, 2, device=dev))
    ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    layer = ops.MxMoELayer(d, wq, device=dev)
    x0 = torch.zeros(w.T, w.H, dtype=torch.bfloat16, device=dev)
    out = layer.forward(x0, torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev),
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not out.any(), "nonzero output for zero activations"
    codes, exps = omx.quantize(np.zeros((w.T, w.H)))
    assert np.array_equal(onv.unpack_codes(to_np(layer.a1_q)), codes)
    assert np.array_equal(to_np(layer.a1_e), exps)


@pytest.mark.parametrize("T,E,k,shared", [(64, 32, 4, 1), (1100, 16, 2, 0)], ids=["decode_like", "three_launch_front"])
def test_mx_layer_dropped_pairs(dev, T, E, k, shared):
    """Half of the routed pairs carry ids outside [0, E) (-1, E, E + 100):
    dropped, as an expert-parallel share drops the experts it does not own."""
    w = Workload(f"mx_dropped_{T}", T, 256, 128, E, k, shared, 0.0, 0.02, 0.01, 1060 + T)
    ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    rng = np.random.default_rng(w.seed)
    bad = rng.choice(np.array([-1, E, E + 100], dtype=np.int32), ids.shape)
    ids = np.where(rng.random(ids.shape) < 0.5, bad, ids).astype(np.int32)
    _judge(MxCase(w, dev, routing=(ids, tw)), dev)

