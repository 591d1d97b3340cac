"""GPU parity of the expert GEMMs and the whole layer (gates G2 and G3).

Stage tests feed oracle-produced inputs into one GPU stage and compare its
output with the oracle's.  Layer tests run the whole product path on the
GPU and compare with the oracle: on every token for shapes that span several
tiles with ragged tails, on sampled tokens at the full workload sizes (in the
same launch configuration the benchmark times).
"""
import time

import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs import Workload
from nvfp4_block_scaled_03_amd import ops
from oracle import moe as omoe
from oracle import nvfp4 as onv
from oracle import routing as oroute

from parity import (bf16_bits, check_a2_bf16, check_a2_nvfp4, check_layer_out, device, relf,
                    to_np)

pytestmark = pytest.mark.gpu

# Small shapes that exercise each tile height (16/32/64/128 rows), several
# column blocks and ragged last tiles; the last one has a shared expert.
SMALL = [
    Workload("s16", 40, 256, 256, 8, 2, 0, 0.0, 0.02, 0.01, 11),
    Workload("s32", 100, 256, 128, 8, 2, 0, 0.0, 0.02, 0.01, 12),
    Workload("s64", 200, 512, 256, 6, 2, 0, 0.5, 0.02, 0.01, 13),
    Workload("s128", 600, 256, 384, 4, 2, 1, 0.0, 0.02, 0.01, 14),
    # odd chunk counts (K = 384, 640) and a GEMM2 width (384) that leaves half
    # of the last 256-column block idle
    Workload("s128b", 300, 384, 640, 3, 1, 0, 0.0, 0.02, 0.01, 15),
]


@pytest.fixture(scope="module")
def dev():
    return device()


class Case:
    """Inputs of one workload on the GPU plus the oracle's view of them.

    The W4A4 oracle runs once, over the pairs of ``tokens`` (all tokens when
    None), and calibrates the static intermediate scale g2 from its own FP64
    h on the way (g2 is then fed to the GPU); the W4A16 oracle runs when first
    asked for."""

    def __init__(self, w: Workload, dev, tokens=None):
        self.w = w
        self.d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
        self.x = moe_inputs.activations(w, device=dev)
        z = moe_inputs.router_logits(w, device=dev)
        ids, tw = oroute.route_topk(to_np(z), w.topk)
        self._setup(w, dev, ids, tw, tokens)

    def _setup(self, w, dev, ids, tw, tokens):
        self.ids_np, self.tw_np = ids, tw
        self.ids = torch.from_numpy(ids).to(dev)
        self.tw = torch.from_numpy(tw).to(dev)
        self.w13 = moe_inputs.expert_weights(w, 13, device=dev)
        self.w2 = moe_inputs.expert_weights(w, 2, device=dev)
        self.ew = omoe.ExpertWeights(lambda e: to_np(self.w13[e]), lambda e: to_np(self.w2[e]))
        self.xf = to_np(self.x).astype(np.float64)
        self.tokens = tokens
        self._ref = {}
        t0 = time.time()
        self._ref["w4a4"] = omoe.layer(self.xf, ids, tw, self.ew, w.E, w.I, variant="w4a4",
                                       shared=w.shared, tokens=tokens, calibrate=True)
        self.g2 = self._ref["w4a4"].g2
        print(f"  oracle {w.name} w4a4: {time.time() - t0:.1f} s", flush=True)
        self.wq = ops.quantize_expert_weights(self.d, self.w13, self.w2, keep_canonical=False)

    def set_g2(self, g2):
        """Use another intermediate scale (drops the cached oracle results)."""
        self.g2 = np.float32(g2)
        self._ref = {}

    def oracle(self, variant):
        if variant not in self._ref:
            print(f"  oracle {self.w.name} {variant}", flush=True)
            self._ref[variant] = omoe.layer(self.xf, self.ids_np, self.tw_np, self.ew, self.w.E,
                                            self.w.I, variant=variant, g2=self.g2,
                                            shared=self.w.shared, tokens=self.tokens)
        return self._ref[variant]


# Full-size cases are built once per module and shared by the tests that need
# them (one at a time, to bound host and device memory).
_CASE = {}


def cached_case(name, dev, tokens=None):
    key = (name, None if tokens is None else tuple(int(t) for t in tokens))
    if key not in _CASE:
        _CASE.clear()
        torch.cuda.empty_cache()
        _CASE[key] = Case(moe_inputs.WORKLOADS[name], dev, tokens=tokens)
    return _CASE[key]


def _uploaded_weights(case: Case, dev):
    """Expert weights quantised by the oracle, prepared by the library."""
    S = case.w.n_experts
    q13 = np.stack([onv.pack_codes(case.ew.quantized(13, e)[0]) for e in range(S)])
    s13 = np.stack([case.ew.quantized(13, e)[1] for e in range(S)])
    g13 = np.array([case.ew.quantized(13, e)[2] for e in range(S)], dtype=np.float32)
    q2 = np.stack([onv.pack_codes(case.ew.quantized(2, e)[0]) for e in range(S)])
    s2 = np.stack([case.ew.quantized(2, e)[1] for e in range(S)])
    g2 = np.array([case.ew.quantized(2, e)[2] for e in range(S)], dtype=np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return ops.ExpertWeights(t(q13), t(s13), t(g13), t(q2), t(s2), t(g2),
                             ops.prep_weights(case.d, 13, t(q13), t(s13)),
                             ops.prep_weights(case.d, 2, t(q2), t(s2)))


# ---------------------------------------------------------------- layout
def _scale_group(kc):
    return next(g for g in (4, 3, 2, 1) if kc % g == 0)


@pytest.mark.parametrize("S,I,H", [(3, 128, 256), (2, 384, 512), (1, 768, 2048)])
def test_prep_layout(dev, S, I, H):
    """The streaming layout is the documented permutation of the canonical
    bytes (chunk counts 1, 2, 3, 4 and 16: every scale group size)."""
    d = ops.dims(4, 1, S, H, I, 0)
    rng = np.random.default_rng(S + I)
    for which, N, K in ((13, 2 * I, H), (2, H, I)):
        q = rng.integers(0, 256, (S, N, K // 2), dtype=np.uint8)
        sf = rng.integers(0, 127, (S, N, K // 16), dtype=np.uint8)
        prep = to_np(ops.prep_weights(d, which, torch.from_numpy(q).to(dev), torch.from_numpy(sf).to(dev)))
        NT, KC = N // 16, K // 128
        G = _scale_group(KC)
        codes = prep[:S * N * K // 2].reshape(S, NT, KC, 64, 16)
        # scales: [S][tile pairs][chunk groups][lanes][G chunks][2 tiles][2 bytes]
        scales = prep[S * N * K // 2:].reshape(S, NT // 2, KC // G, 64, G, 2, 2)
        nt = np.arange(NT)[:, None]
        n = np.arange(64)[None, :] % 16
        g = np.arange(64)[None, :] // 16
        row = np.where(nt % 2 == 1, I + 16 * (nt // 2) + n, 16 * (nt // 2) + n) if which == 13 \
            else nt * 16 + n                                   # [NT][64]
        for kc in range(KC):
            want_q = q[:, row[..., None], kc * 64 + 16 * g[..., None] + np.arange(16)]
            assert np.array_equal(codes[:, :, kc], want_q), (which, kc)
            want_s = sf[:, row[..., None], kc * 8 + 2 * g[..., None] + np.arange(2)]   # [S][NT][64][2]
            got_s = scales[:, :, kc // G, :, kc % G].transpose(0, 1, 3, 2, 4).reshape(S, NT, 64, 2)
            assert np.array_equal(got_s, want_s), (which, kc)


# ---------------------------------------------------------------- stages
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_gemm1_w4a4_stage(dev, w):
    case = Case(w, dev)
    ref = case.oracle("w4a4")
    wq = _uploaded_weights(case, dev)
    al = ops.moe_align(case.d, case.ids)
    a1_q = torch.from_numpy(onv.pack_codes(ref.a1_codes)).to(dev)
    a1_sf = torch.from_numpy(ref.a1_scales).to(dev)
    g1 = torch.tensor([float(ref.g1)], device=dev)
    g2 = torch.tensor([float(case.g2)], device=dev)
    rows = ref.rows
    # Codes in (decoded in the kernels), then the exact f16 copy in (decoded
    # once, by the oracle here); both must give a2 to the same bar, and the
    # a2 copy must be the exact decoding of the a2 codes it accompanies.
    a2_q, a2_sf = ops.gemm1_w4a4(case.d, a1_q, a1_sf, g1, al, wq, g2)
    chk = check_a2_nvfp4(to_np(a2_q)[rows], to_np(a2_sf)[rows], ref.h, case.g2, what=f"{w.name} stage")
    print(f"{w.name}: a2 exact={chk.exact} flips={chk.flips} of {ref.h.size}")
    a1_deq = torch.from_numpy(onv.dequantize(ref.a1_codes, ref.a1_scales, 1.0)).to(dev).to(torch.float16)
    a2_deq = torch.empty(w.pairs, w.I, dtype=torch.float16, device=dev)
    b2_q, b2_sf = ops.gemm1_w4a4(case.d, None, None, g1, al, wq, g2, a1_deq=a1_deq, a2_deq=a2_deq)
    chk2 = check_a2_nvfp4(to_np(b2_q)[rows], to_np(b2_sf)[rows], ref.h, case.g2,
                          what=f"{w.name} stage")
    got_codes = onv.unpack_codes(to_np(b2_q)[rows])
    assert np.array_equal(to_np(a2_deq)[rows].astype(np.float64),
                          onv.dequantize(got_codes, to_np(b2_sf)[rows], 1.0))
    print(f"{w.name} (decoded a1): a2 exact={chk2.exact} flips={chk2.flips} of {ref.h.size}")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_gemm2_w4a4_stage(dev, w):
    case = Case(w, dev)
    ref = case.oracle("w4a4")
    wq = _uploaded_weights(case, dev)
    al = ops.moe_align(case.d, case.ids)
    P = w.pairs
    a2_q = torch.zeros(P, w.I // 2, dtype=torch.uint8, device=dev)
    a2_sf = torch.zeros(P, w.I // 16, dtype=torch.uint8, device=dev)
    a2_q[torch.from_numpy(ref.rows).to(dev)] = torch.from_numpy(onv.pack_codes(ref.a2_codes)).to(dev)
    a2_sf[torch.from_numpy(ref.rows).to(dev)] = torch.from_numpy(ref.a2_scales).to(dev)
    g2 = torch.tensor([float(case.g2)], device=dev)
    out32 = ops.gemm2_w4a4(case.d, a2_q, a2_sf, g2, al, case.tw, wq, out_dtype=torch.float32)
    out16 = ops.gemm2_w4a4(case.d, a2_q, a2_sf, g2, al, case.tw, wq, out_dtype=torch.bfloat16)
    got = to_np(out32).astype(np.float64)
    check_layer_out(got, ref.out, f"{w.name} gemm2")
    assert torch.equal(out16, out32.to(torch.bfloat16))
    # The same a2 as its exact f16 copy (codes not passed).
    a2_deq = torch.zeros(P, w.I, dtype=torch.float16, device=dev)
    a2_deq[torch.from_numpy(ref.rows).to(dev)] = torch.from_numpy(
        onv.dequantize(ref.a2_codes, ref.a2_scales, 1.0)).to(dev).to(torch.float16)
    outd = ops.gemm2_w4a4(case.d, None, None, g2, al, case.tw, wq, out_dtype=torch.float32, a2_deq=a2_deq)
    check_layer_out(to_np(outd).astype(np.float64), ref.out, f"{w.name} gemm2 (decoded a2)")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_w4a16_stages(dev, w):
    case = Case(w, dev)
    ref = case.oracle("w4a16")
    wq = _uploaded_weights(case, dev)
    al = ops.moe_align(case.d, case.ids)
    a2 = ops.gemm1_w4a16(case.d, case.x, al, wq)
    check_a2_bf16(bf16_bits(a2)[ref.rows], ref.h, what=f"{w.name} stage")
    a2_in = torch.zeros(w.pairs, w.I, dtype=torch.bfloat16, device=dev)
    a2_in[torch.from_numpy(ref.rows).to(dev)] = torch.from_numpy(ref.a2_bf16).to(dev).to(torch.bfloat16)
    out32 = ops.gemm2_w4a16(case.d, a2_in, al, case.tw, wq, out_dtype=torch.float32)
    check_layer_out(to_np(out32).astype(np.float64), ref.out, f"{w.name} w4a16 gemm2")


# ---------------------------------------------------------------- whole layer
def _run_layer(case: Case, dev, variant, decoded_copies=None, side_stream=None):
    g2 = torch.tensor([float(case.g2)], device=dev)
    layer = ops.MoELayer(case.d, case.wq, g2, device=dev, decoded_copies=decoded_copies,
                         side_stream=side_stream)
    out32 = layer.forward(case.x, case.ids, case.tw, variant, out_dtype=torch.float32).clone()
    out16 = layer.forward(case.x, case.ids, case.tw, variant, out_dtype=torch.bfloat16).clone()
    torch.cuda.synchronize()
    return layer, out32, out16


def _judge_layer(case: Case, dev, variant, decoded_copies=None, run=None):
    ref = case.oracle(variant)
    layer, out32, out16 = run if run is not None else _run_layer(case, dev, variant, decoded_copies)
    assert torch.equal(out16, out32.to(torch.bfloat16)), "bf16 output != bf16(f32 output)"
    toks = np.arange(case.w.T) if case.tokens is None else np.asarray(case.tokens)
    rows = ref.rows
    if variant == "w4a4":
        # a1 is exact; a2 may differ only at near ties (validated), and the
        # expected output is then the oracle's down projection of that a2.
        assert np.array_equal(to_np(layer.a1_q), onv.pack_codes(ref.a1_codes))
        assert np.array_equal(to_np(layer.a1_sf), ref.a1_scales)
        if layer.a1_deq is not None:
            assert np.array_equal(to_np(layer.a1_deq).astype(np.float64),
                                  onv.dequantize(ref.a1_codes, ref.a1_scales, 1.0))
        chk = check_a2_nvfp4(to_np(layer.a2_q)[rows], to_np(layer.a2_sf)[rows], ref.h, case.g2,
                             what=f"{case.w.name} layer")
        if layer.a2_deq is not None:
            assert np.array_equal(to_np(layer.a2_deq)[rows].astype(np.float64),
                                  onv.dequantize(chk.codes, chk.scales, 1.0))
        exp = ref.out if chk.exact else omoe.down_and_combine(
            onv.dequantize(chk.codes, chk.scales, case.g2), rows, ref.sorted_pair, ref.offsets,
            case.tw_np, case.ew, case.w.T, case.w.topk)
    else:
        got_a2 = check_a2_bf16(bf16_bits(layer.a2_bf16)[rows], ref.h, what=f"{case.w.name} layer")
        exp = ref.out if np.array_equal(got_a2, ref.a2_bf16) else omoe.down_and_combine(
            got_a2, rows, ref.sorted_pair, ref.offsets, case.tw_np, case.ew, case.w.T, case.w.topk)
    got = to_np(out32).astype(np.float64)[toks]
    rf, ma = check_layer_out(got, exp[toks], f"{case.w.name} {variant}")
    e2e = relf(got, ref.out[toks])
    assert e2e <= 2e-3, f"end-to-end rel-F {e2e:.2e}"
    print(f"{case.w.name} {variant}: relF {rf:.2e} maxabs/rms {ma:.2e} (vs own-a2 oracle {e2e:.2e})")


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
@pytest.mark.parametrize("w", SMALL + [moe_inputs.WORKLOADS["tiny"]], ids=lambda w: w.name)
def test_layer_small(dev, w, variant):
    _judge_layer(Case(w, dev), dev, variant)


@pytest.mark.parametrize("decoded", [True, False], ids=["decoded", "codes"])
@pytest.mark.parametrize("w", SMALL + [moe_inputs.WORKLOADS["tiny"]], ids=lambda w: w.name)
def test_layer_small_activation_paths(dev, w, decoded):
    """W4A4 with the GEMMs reading the exact f16 activation copies, and with
    them decoding the codes themselves."""
    _judge_layer(Case(w, dev), dev, "w4a4", decoded_copies=decoded)


# Full-size workloads, in the launch configuration the benchmark times.  At
# decode and large_e every token is compared (large_e: all 256 shared-expert
# rows too); at prefill and skew a sample of tokens is compared end to end and
# every row of the hottest expert and of the last expert is compared at a2.
FULL_EVERY = [("decode", "w4a4", None), ("decode", "w4a4", True), ("decode", "w4a16", None),
              ("large_e", "w4a4", None), ("large_e", "w4a4", False), ("large_e", "w4a16", None)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,variant,decoded", FULL_EVERY, ids=lambda v: str(v))
def test_layer_full_size_every_token(dev, name, variant, decoded):
    print(f"full-size {name} {variant} decoded={decoded}", flush=True)
    case = cached_case(name, dev)
    _judge_layer(case, dev, variant, decoded)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
def test_layer_full_size_two_streams(dev, variant):
    """The 512-expert layer as the benchmark runs it: the tall experts' GEMM1
    and GEMM2 on a second stream beside the short experts', joined before the
    combine; every token judged against the oracle."""
    print(f"full-size large_e {variant} two streams", flush=True)
    case = cached_case("large_e", dev)
    run = _run_layer(case, dev, variant, side_stream=torch.cuda.Stream())
    assert run[0].side is not None
    _judge_layer(case, dev, variant, run=run)


def _rows_of(case, e):
    off = case.oracle("w4a4").offsets
    return np.arange(off[e], off[e + 1])


FULL_SAMPLED = [("prefill", "w4a4", None), ("prefill", "w4a4", False), ("prefill", "w4a16", None),
                ("skew", "w4a4", None), ("skew", "w4a16", None)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,variant,decoded", FULL_SAMPLED, ids=lambda v: str(v))
def test_layer_full_size_hot_and_last_experts(dev, name, variant, decoded):
    """Sampled tokens end to end; every row of the hottest and of the last
    non-empty expert at a2 (their last tiles are the last ones the GEMM
    kernels dispatch, at the largest row offsets).  g2 is calibrated over all
    the rows compared."""
    print(f"full-size {name} {variant} decoded={decoded}", flush=True)
    w = moe_inputs.WORKLOADS[name]
    toks = np.sort(np.random.default_rng(w.seed).choice(w.T, 12, replace=False))
    case = cached_case(name, dev, tokens=toks)
    off = case.oracle("w4a4").offsets
    counts = np.diff(off)
    hot, last = int(np.argmax(counts)), int(np.nonzero(counts)[0][-1])
    sp = case.oracle("w4a4").sorted_pair
    x_hat = omoe.activations_hat(case.xf, variant)[3]
    h = {}
    for e in sorted({hot, last}):
        tok, _ = omoe.pair_token_weight(sp[off[e]:off[e + 1]], w.T, w.topk, case.tw_np)
        h[e] = omoe.expert_h(x_hat, tok, case.ew, e, w.I)
    if variant == "w4a4":
        g2 = max(float(case.oracle("w4a4").g2), *[float(onv.global_scale(v)) for v in h.values()])
        if np.float32(g2) != case.g2:
            case.set_g2(g2)
    print(f"  hot expert {hot} ({counts[hot]} rows), last expert {last} ({counts[last]} rows)", flush=True)
    run = _run_layer(case, dev, variant, decoded)
    layer = run[0]
    for e, he in h.items():
        rows = np.arange(off[e], off[e + 1])
        if variant == "w4a4":
            check_a2_nvfp4(to_np(layer.a2_q)[rows], to_np(layer.a2_sf)[rows], he, case.g2,
                           what=f"{name} expert rows")
        else:
            check_a2_bf16(bf16_bits(layer.a2_bf16)[rows], he, what=f"{name} expert rows")
    _judge_layer(case, dev, variant, decoded, run=run)


# The largest batch the tests run through the whole layer: 32768 tokens,
# 262144 pairs (256 chunks of pairs, past the scan's register path), about
# 2100 tiles of 128 rows per GEMM, a 2 GiB FP32 workspace (the combine's
# non-temporal path) and activation offsets up to 2^27.
_MAX_ROWS = Workload("max_rows", 32768, 2048, 768, 128, 8, 0, 0.0, 0.02, 0.01, 1007)


@pytest.mark.timeout(900)
def test_layer_max_rows_sampled(dev):
    """The W4A4 layer at 32768 tokens: a1 bit for bit over every token, a2
    and the output at the first, the last and 10 sampled tokens."""
    print("max-rows layer", flush=True)
    _CASE.clear()
    torch.cuda.empty_cache()
    w = _MAX_ROWS
    rng = np.random.default_rng(w.seed)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 10, replace=False)]))
    case = Case(w, dev, tokens=toks)
    _judge_layer(case, dev, "w4a4")
    del case
    torch.cuda.empty_cache()


def test_layer_is_deterministic(dev):
    case = Case(moe_inputs.WORKLOADS["decode"], dev, tokens=[0])
    _, a, _ = _run_layer(case, dev, "w4a4")
    _, b, _ = _run_layer(case, dev, "w4a4")
    assert torch.equal(a, b)


# ---------------------------------------------------------------- ragged tiles
# Rows per expert chosen so that the last 128-row tile of the experts falls in
# every class of active 16-row groups of the wide kernel (1, 2, 4 and 8 groups,
# each at both ends of its range), plus an empty expert; top-1 routing in a
# seeded order, so the tokens of an expert are scattered over the batch.
RAGGED_COUNTS = [1, 16, 17, 32, 33, 64, 65, 128, 129, 0, 200, 255, 256, 257, 300]


class RoutedCase(Case):
    """Case with routing given by expert row counts instead of router logits."""

    def __init__(self, counts, dev, H=256, I=128, seed=71):
        E = len(counts)
        w = Workload("ragged", int(sum(counts)), H, I, E, 1, 0, 0.0, 0.02, 0.01, seed)
        ids = np.repeat(np.arange(E, dtype=np.int32), counts)
        ids = ids[np.random.default_rng(seed).permutation(ids.size)].reshape(-1, 1)
        self.w = w
        self.d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
        self.x = moe_inputs.activations(w, device=dev)
        self._setup(w, dev, ids, np.ones((w.T, 1), dtype=np.float32), None)


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
def test_layer_ragged_tile_heights(dev, variant):
    """Every token of a layer whose experts end in tiles of every height class
    of the 128-row kernel (mean rows per expert > 96 selects it; W4A4 with
    the exact f16 activation copies it reads)."""
    case = RoutedCase(RAGGED_COUNTS, dev)
    assert case.w.pairs / case.w.E > 96
    _judge_layer(case, dev, variant, decoded_copies=True if variant == "w4a4" else None)


# Short experts on average (mean 13.7 rows: the streaming regime) but some
# experts hold up to 200 rows: the experts with more than 32 rows run on the
# 128-row kernel, the others on the streaming kernel.
SPLIT_COUNTS = [200, 100, 40, 33, 32, 17, 16, 15, 8, 5, 4, 3, 2, 1, 0, 1] + [3] * 24


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
def test_layer_split_short_and_tall_experts(dev, variant):
    case = RoutedCase(SPLIT_COUNTS, dev, seed=72)
    assert case.w.pairs / case.w.E <= 16 and case.w.T > 64
    _judge_layer(case, dev, variant, decoded_copies=True if variant == "w4a4" else None)


# The largest expert count the boundary takes: 1023 routed experts and a
# shared one (1024 slots).  Short experts on average and the shared expert
# tall, so plan entries and prepared weights of nearly every slot are in
# play, the split launches run (W4A4 with f16 copies, W4A16), or the 16-row
# streaming kernel takes every tile (W4A4 from the codes), and the combine
# adds the shared row of every token.
MAX_EXPERTS = Workload("max_experts", 300, 128, 128, 1023, 4, 1, 0.0, 0.02, 0.01, 1011)


@pytest.fixture(scope="module")
def max_experts_case(dev):
    return Case(MAX_EXPERTS, dev)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant,decoded", [("w4a4", True), ("w4a4", False), ("w4a16", None)],
                         ids=["w4a4-f16-copies", "w4a4-codes", "w4a16"])
def test_layer_max_experts(dev, max_experts_case, variant, decoded):
    case = max_experts_case
    assert case.w.E + case.w.shared == 1024
    _judge_layer(case, dev, variant, decoded_copies=decoded)


# Batch-one decode and a three-token batch: every tile holds a single row,
# the front end runs one quantising workgroup, the combine one or three
# tokens.
FEW_TOKENS = [Workload("one_token", 1, 256, 128, 128, 8, 0, 0.0, 0.02, 0.01, 1021),
              Workload("three_tokens", 3, 256, 128, 64, 6, 1, 0.0, 0.02, 0.01, 1022)]


@pytest.mark.parametrize("variant,decoded", [("w4a4", True), ("w4a4", False), ("w4a16", None)],
                         ids=["w4a4-f16-copies", "w4a4-codes", "w4a16"])
@pytest.mark.parametrize("w", FEW_TOKENS, ids=lambda w: w.name)
def test_layer_few_tokens(dev, w, variant, decoded):
    _judge_layer(Case(w, dev), dev, variant, decoded_copies=decoded)


@pytest.mark.parametrize("variant,decoded", [("w4a4", True), ("w4a4", False), ("w4a16", None)],
                         ids=["w4a4-f16-copies", "w4a4-codes", "w4a16"])
@pytest.mark.parametrize("T", [40, 1100], ids=["one_launch_front", "three_launch_front"])
def test_layer_zero_activations(dev, T, variant, decoded):
    """All-zero activations (the oracle's result is pinned to exact zeros on
    the CPU): g1 = 0, zero codes, scales and f16 copy, and an exactly zero
    output.  1100 tokens x 256 take the three-launch front end."""
    w = Workload("zeros", T, 256, 128, 16, 2, 1, 0.0, 0.02, 0.01, 1041)
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    wq = ops.quantize_expert_weights(d, moe_inputs.expert_weights(w, 13, device=dev),
                                     moe_inputs.expert_weights(w, 2, device=dev), keep_canonical=False)
    ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
    layer = ops.MoELayer(d, wq, torch.tensor([0.003], device=dev), device=dev, decoded_copies=decoded)
    x0 = torch.zeros(w.T, w.H, dtype=torch.bfloat16, device=dev)
    out = layer.forward(x0, torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev), variant,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not out.any(), "nonzero output for zero activations"
    if variant == "w4a4":
        assert float(layer.g1.item()) == 0.0
        assert not layer.a1_q.any() and not layer.a1_sf.any()
        if layer.a1_deq is not None:
            assert not layer.a1_deq.any()


def _drop_ids(ids, E, frac, seed):
    """Replace a fraction of the expert ids by ones outside [0, E) (-1, E
    itself, which is the shared slot's index, and E + 100): such pairs are
    dropped, as an expert-parallel share drops the experts it does not own."""
    rng = np.random.default_rng(seed)
    bad = rng.choice(np.array([-1, E, E + 100], dtype=np.int32), ids.shape)
    return np.where(rng.random(ids.shape) < frac, bad, ids).astype(np.int32)


class DroppedCase(Case):
    def __init__(self, w: Workload, dev, frac, seed):
        self.w = w
        self.d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
        self.x = moe_inputs.activations(w, device=dev)
        ids, tw = oroute.route_topk(to_np(moe_inputs.router_logits(w, device=dev)), w.topk)
        self._setup(w, dev, _drop_ids(ids, w.E, frac, seed), tw, None)


DROPPED = [Workload("dropped_decode", 64, 256, 128, 32, 4, 1, 0.0, 0.02, 0.01, 1051),
           Workload("dropped_big", 1100, 256, 128, 16, 2, 0, 0.0, 0.02, 0.01, 1052)]


@pytest.mark.parametrize("variant,decoded", [("w4a4", True), ("w4a4", False), ("w4a16", None)],
                         ids=["w4a4-f16-copies", "w4a4-codes", "w4a16"])
@pytest.mark.parametrize("w", DROPPED, ids=lambda w: w.name)
def test_layer_dropped_pairs(dev, w, variant, decoded):
    """Half of the routed pairs carry ids outside [0, E): they get no row,
    their inverse position is -1, and the combine leaves them out (a token
    may keep only its shared row, or nothing)."""
    case = DroppedCase(w, dev, 0.5, w.seed)
    al = ops.moe_align(case.d, case.ids)
    off, sp, inv = omoe.align(case.ids_np, w.E, w.shared)
    assert off[-1] < w.pairs
    assert np.array_equal(to_np(al.offsets), off)
    assert np.array_equal(to_np(al.sorted_pair)[:off[-1]], sp)
    assert np.array_equal(to_np(al.inv_pos), inv)
    _judge_layer(case, dev, variant, decoded_copies=decoded)


# 262144 pairs with I = 4096: the down projection's 16-bit activation rows
# span 2^31 bytes, past the 32-bit buffer offsets of the streaming and wide
# kernels, so it runs on the LDS-staged kernel with 64-bit addressing (f16
# copy or bf16), while the 4-bit codes still fit.
_WIDE_OFFSETS = Workload("wide_offsets", 32768, 128, 4096, 8, 8, 0, 0.0, 0.02, 0.01, 1071)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant,decoded", [("w4a4", True), ("w4a4", False), ("w4a16", None)],
                         ids=["w4a4-f16-copies", "w4a4-codes", "w4a16"])
def test_layer_wide_offsets_sampled(dev, variant, decoded):
    w = _WIDE_OFFSETS
    assert w.pairs * w.I * 2 >= 2 ** 31
    _CASE.clear()
    torch.cuda.empty_cache()
    rng = np.random.default_rng(w.seed)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 10, replace=False)]))
    case = Case(w, dev, tokens=toks)
    _judge_layer(case, dev, variant, decoded_copies=decoded)
    del case
    torch.cuda.empty_cache()

