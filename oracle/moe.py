"""Expert-path reference: permutation by expert and the NVFP4 MoE layer.

FP64 NumPy, test infrastructure only.  What the pages fix:

* The expert GEMMs are grouped per expert, with per-expert problem sizes kept
  on the device and the tokens permuted by expert beforehand (the grouped-GEMM
  metadata step ``get_cutlass_moe_mm_data`` and the device-resident problem
  shapes in vLLM PR #29242, commit list and debug trace).
* Each expert's GEMM output is scaled by one FP32 alpha per expert with no C
  input (``alpha_ptr_array`` with ``beta = 0``, vLLM PR #29242, review of
  ``nvfp4_blockwise_moe_kernel.cu``).
* The layer output is bfloat16 ("Force bf16 only", vLLM PR #29242 commits).
* The emulation backend dequantises NVFP4 weights to higher precision,
  quantise-dequantises the activations and runs the expert MLP in high
  precision (vLLM PR #35737, "Purpose"); this module does the same in FP64.
* A grouped GEMM can be wrong while the dense one is right (FlashInfer #2723,
  "The Problem"), so ``bruteforce.py`` recomputes the layer token by token.

Readings where the pages are silent:

* w13 rows [0, I) are the gate projection and rows [I, 2I) the up
  projection; h = silu(gate) * up with silu(z) = z / (1 + exp(-z)).
* alpha1[e] = g1 * gw13[e] and alpha2[e] = g2 * gw2[e]: the product of the
  activation and weight global scales.  Here the dequantised values carry their
  own global scales, which is the same product taken in exact arithmetic.
* The intermediate h is requantised to NVFP4 with a static global scale g2
  that the caller supplies (one scalar per layer).
* The router weight multiplies the down-projection output in FP32/FP64, not h.
* The shared expert, when present, is expert slot E: every token visits it
  with weight 1 as pseudo-pair f = T*k + t.
* W4A16: activations stay bfloat16, weights are dequantised, and the
  intermediate h is rounded to bfloat16 instead of NVFP4.
* (token, expert) pairs are numbered f = t*k + j; pairs are ordered by expert,
  and by f within an expert.  Pairs whose expert id is outside [0, E) are
  dropped: they get no row and inverse position -1.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np

from . import nvfp4


# --------------------------------------------------------------------------
# Permutation by expert.
# --------------------------------------------------------------------------
def align(topk_ids, n_routed: int, shared: int = 0):
    """Return (offsets int32 [E+shared+1], sorted_pair int32 [P], inv_pos int32 [P]).

    ``sorted_pair[p]`` is the pair index f placed at row p; rows of expert e
    are ``offsets[e] <= p < offsets[e+1]``; ``inv_pos[f]`` is the row of pair f
    (or -1 for a dropped pair).  P = T*k + shared*T.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    expert_of = ids.reshape(-1)
    if shared:
        expert_of = np.concatenate([expert_of, np.full(T, n_routed, dtype=np.int64)])
    n_slots = n_routed + (1 if shared else 0)
    valid = (expert_of >= 0) & (expert_of < n_routed)
    if shared:
        valid[T * k:] = True
    key = np.where(valid, expert_of, n_slots)
    order = np.argsort(key, kind="stable")
    n_valid = int(valid.sum())
    sorted_pair = order[:n_valid]
    counts = np.bincount(expert_of[valid], minlength=n_slots)[:n_slots]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv_pos = np.full(expert_of.shape[0], -1, dtype=np.int64)
    inv_pos[sorted_pair] = np.arange(n_valid)
    return offsets.astype(np.int32), sorted_pair.astype(np.int32), inv_pos.astype(np.int32)


def pair_token_weight(f, T: int, k: int, topk_w):
    """Token index and router weight of pair indices ``f`` (shared pairs: weight 1)."""
    f = np.asarray(f, dtype=np.int64)
    routed = f < T * k
    tok = np.where(routed, f // k, f - T * k)
    w = np.ones(f.shape, dtype=np.float64)
    tw = np.asarray(topk_w, dtype=np.float64).reshape(-1)
    w[routed] = tw[f[routed]]
    return tok, w


# --------------------------------------------------------------------------
# Expert weights, quantised on demand from FP32.
# --------------------------------------------------------------------------
class ExpertWeights:
    """NVFP4 expert weights with one global scale per expert matrix.

    ``src13(e)`` returns the FP32 [2I, H] gate/up weight of expert slot e and
    ``src2(e)`` the FP32 [H, I] down weight.  Each matrix is quantised with
    ``nvfp4.quantize`` along its contraction dimension the first time it is
    needed.
    """

    def __init__(self, src13: Callable[[int], np.ndarray], src2: Callable[[int], np.ndarray]):
        self._src = {13: src13, 2: src2}
        self._cache: dict = {}

    @classmethod
    def from_arrays(cls, w13, w2):
        w13 = np.asarray(w13, dtype=np.float32)
        w2 = np.asarray(w2, dtype=np.float32)
        return cls(lambda e: w13[e], lambda e: w2[e])

    def quantized(self, which: int, e: int):
        """(codes uint8 [N, K], scales uint8 [N, K/16], g float32)."""
        key = (which, int(e))
        if key not in self._cache:
            w = np.asarray(self._src[which](int(e)), dtype=np.float32)
            g = nvfp4.global_scale(w)
            codes, scales = nvfp4.quantize(w, g)
            self._cache[key] = (codes, scales, g)
        return self._cache[key]

    def dequantized(self, which: int, e: int) -> np.ndarray:
        codes, scales, g = self.quantized(which, e)
        return nvfp4.dequantize(codes, scales, g)

    def drop(self, which: int, e: int) -> None:
        """Forget the quantisation of one matrix (to bound host memory)."""
        self._cache.pop((which, int(e)), None)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(c, I: int):
    """h = silu(gate) * up for c = [gate | up] along the last axis."""
    return silu(c[..., :I]) * c[..., I:]


def expert_h(x_hat, tok, weights: "ExpertWeights", e: int, I: int) -> np.ndarray:
    """FP64 SwiGLU intermediate of expert slot e for the rows of tokens ``tok``:
    h = swiglu(x_hat[tok] W13_e^T)."""
    return swiglu(np.asarray(x_hat)[np.asarray(tok)] @ weights.dequantized(13, e).T, I)


def activations_hat(x, variant: str):
    """(g1, codes, scales, x_hat): the dequantised W4A4 activations, or x
    itself for W4A16 (g1, codes, scales None)."""
    x = np.asarray(x, dtype=np.float64)
    if variant == "w4a4":
        g1 = nvfp4.global_scale(x)
        codes, scales = nvfp4.quantize(x, g1)
        return g1, codes, scales, nvfp4.dequantize(codes, scales, g1)
    return None, None, None, x


# --------------------------------------------------------------------------
# The layer.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LayerResult:
    out: np.ndarray                # FP64 [T, H] (rows of unselected tokens are 0)
    offsets: np.ndarray
    sorted_pair: np.ndarray
    inv_pos: np.ndarray
    g1: Optional[np.float32]       # activation global scale (W4A4)
    a1_codes: Optional[np.ndarray]  # uint8 [T, H] (W4A4)
    a1_scales: Optional[np.ndarray]  # uint8 [T, H/16] (W4A4)
    rows: np.ndarray               # sorted rows p that were computed
    h: np.ndarray                  # FP64 [len(rows), I] pre-requantisation intermediate
    a2_codes: Optional[np.ndarray]  # uint8 [len(rows), I] (W4A4)
    a2_scales: Optional[np.ndarray]  # uint8 [len(rows), I/16] (W4A4)
    a2_bf16: Optional[np.ndarray]   # FP64 [len(rows), I] bfloat16 values (W4A16)
    d: np.ndarray                  # FP64 [len(rows), H] down-projection output per row
    g2: Optional[np.float32] = None  # intermediate global scale used (W4A4)


def layer(x, topk_ids, topk_w, weights: ExpertWeights, n_routed: int, I: int,
          variant: str = "w4a4", g2=None, shared: int = 0, tokens=None,
          calibrate: bool = False) -> LayerResult:
    """One mixture-of-experts expert layer.

    x: [T, H] bf16 values (any float dtype holding them); topk_ids int [T, k];
    topk_w float32 [T, k]; g2: FP32 intermediate global scale (W4A4 only).
    ``tokens`` restricts the computation to the pairs of those tokens (the
    activation global scale is still taken over all of x).  ``calibrate``
    (W4A4): take g2 = fl32(max |h| / 2688) over the computed pairs (the value
    ``calibrate_g2`` returns for the same tokens) instead of the argument; the
    result's ``g2`` field holds the value used.
    """
    if variant not in ("w4a4", "w4a16"):
        raise ValueError(variant)
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    k = np.asarray(topk_ids).shape[1]
    offsets, sorted_pair, inv_pos = align(topk_ids, n_routed, shared)
    g1, a1_codes, a1_scales, x_hat = activations_hat(x, variant)
    keep_tok = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    out = np.zeros((T, H), dtype=np.float64)
    rows_all, h_all, a2c_all, a2s_all, a2b_all, d_all = [], [], [], [], [], []
    # GEMM1 + SwiGLU of every expert first (g2 may depend on all of them).
    stage1 = []
    for e in range(len(offsets) - 1):
        rows = np.arange(offsets[e], offsets[e + 1])
        tok, wgt = pair_token_weight(sorted_pair[rows], T, k, topk_w)
        sel = keep_tok[tok]
        rows, tok, wgt = rows[sel], tok[sel], wgt[sel]
        if rows.size == 0:
            continue
        stage1.append((e, rows, tok, wgt, expert_h(x_hat, tok, weights, e, I)))
    if calibrate and variant == "w4a4":
        amax = max((float(np.abs(h).max()) for *_, h in stage1), default=0.0)
        g2 = np.float32(amax / (nvfp4.E2M1_MAX * nvfp4.E4M3_MAX))
    for e, rows, tok, wgt, h in stage1:
        if variant == "w4a4":
            a2c, a2s = nvfp4.quantize(h, g2)
            h_hat = nvfp4.dequantize(a2c, a2s, g2)
            a2c_all.append(a2c)
            a2s_all.append(a2s)
        else:
            h_hat = nvfp4.round_to_bf16(h)
            a2b_all.append(h_hat)
        d = h_hat @ weights.dequantized(2, e).T
        np.add.at(out, tok, wgt[:, None] * d)
        rows_all.append(rows)
        h_all.append(h)
        d_all.append(d)

    def cat(lst, width):
        return np.concatenate(lst) if lst else np.zeros((0, width))

    return LayerResult(
        out=out, offsets=offsets, sorted_pair=sorted_pair, inv_pos=inv_pos,
        g1=g1, a1_codes=a1_codes, a1_scales=a1_scales, g2=g2,
        rows=np.concatenate(rows_all) if rows_all else np.zeros(0, dtype=np.int64),
        h=cat(h_all, I),
        a2_codes=cat(a2c_all, I).astype(np.uint8) if variant == "w4a4" else None,
        a2_scales=cat(a2s_all, I // 16).astype(np.uint8) if variant == "w4a4" else None,
        a2_bf16=cat(a2b_all, I) if variant == "w4a16" else None,
        d=cat(d_all, H))


def down_and_combine(a2_hat, rows, sorted_pair, offsets, topk_w, weights: ExpertWeights,
                     T: int, k: int) -> np.ndarray:
    """Second half of the layer from a given dequantised intermediate.

    ``a2_hat`` [len(rows), I] are the FP64 values of the requantised
    intermediate at sorted rows ``rows``.  Returns out FP64 [T, H] summed over
    the given rows: out[t] += w * (Ŵ2_e a2_hat).
    """
    rows = np.asarray(rows, dtype=np.int64)
    H = weights.dequantized(2, 0).shape[0]
    out = np.zeros((T, H), dtype=np.float64)
    expert_of_row = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(expert_of_row):
        sel = expert_of_row == e
        tok, wgt = pair_token_weight(sorted_pair[rows[sel]], T, k, topk_w)
        d = a2_hat[sel] @ weights.dequantized(2, int(e)).T
        np.add.at(out, tok, wgt[:, None] * d)
    return out


def calibrate_g2(x, topk_ids, weights: ExpertWeights, n_routed: int, I: int,
                 shared: int = 0, tokens=None) -> np.float32:
    """Static intermediate global scale: fl32(max |h| / 2688) over the layer's
    W4A4 intermediate (or over the pairs of ``tokens``), computed in FP64."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    k = np.asarray(topk_ids).shape[1]
    x_hat = activations_hat(x, "w4a4")[3]
    offsets, sorted_pair, _ = align(topk_ids, n_routed, shared)
    keep_tok = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    amax = 0.0
    for e in range(len(offsets) - 1):
        f = sorted_pair[offsets[e]:offsets[e + 1]]
        tok, _ = pair_token_weight(f, T, k, np.zeros(T * k))
        tok = tok[keep_tok[tok]]
        if tok.size == 0:
            continue
        amax = max(amax, float(np.abs(expert_h(x_hat, tok, weights, e, I)).max()))
    return np.float32(amax / (nvfp4.E2M1_MAX * nvfp4.E4M3_MAX))
