"""OCP MXFP4 reference: E2M1 elements with one E8M0 scale per 32 (FP64 NumPy).

Test infrastructure only (imported by tests/, smoke() and bench.py's CPU
baseline, never by the product path).

The pages name OCP MX as the other block format of the emulation backend
(vLLM PR #35737: MXFP4 / MXFP6 models on MI3xx) but do not spell it out; the
reading taken here is the format's usual definition:

* A block is 32 consecutive elements along the contraction dimension.
* Its scale is the power of two X = 2^(floor(log2 amax) - 2) (2 = the
  exponent of E2M1's largest value 6 = 1.5 * 2^2), stored as the E8M0 byte
  floor(log2 amax) - 2 + 127, clamped to [0, 254]; a block of zeros gets byte
  0.
* Each element is v / X (exact: X is a power of two) rounded to the nearest
  E2M1 value, ties to the even code, magnitudes above 6 saturating at 6, the
  sign kept (negative values that round to 0 encode as 0x8).
* There is no second-level (global) scale.
"""
from __future__ import annotations

import numpy as np

from . import nvfp4

BLOCK = 32
E8M0_BIAS = 127


def block_exponents(x) -> np.ndarray:
    """E8M0 bytes uint8 [..., K/32] of x [..., K]."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("contraction length must be a multiple of 32")
    amax = np.abs(x.reshape(*x.shape[:-1], K // BLOCK, BLOCK)).max(axis=-1)
    # floor(log2 amax), exactly: amax = m * 2^fe with m in [0.5, 1).
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
    e = fe.astype(np.int64) - 1
    code = np.clip(e - 2 + E8M0_BIAS, 0, 254)
    return np.where(amax > 0, code, 0).astype(np.uint8)


def encode(x, exps) -> np.ndarray:
    """E2M1 codes uint8 [..., K] of x given its block exponent bytes."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    blocks = x.reshape(*x.shape[:-1], K // BLOCK, BLOCK)
    scale = np.ldexp(1.0, np.asarray(exps, dtype=np.int64) - E8M0_BIAS)[..., None]
    r = np.abs(blocks) / scale                       # exact (power of two)
    mag = nvfp4.round_quotient_to_grid(r, np.float64(1.0), nvfp4.E2M1_MAGS)
    sign = np.signbit(blocks).astype(np.int64)
    return (mag | (sign << 3)).reshape(x.shape).astype(np.uint8)


def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """(codes uint8 [..., K] values 0..15, exponent bytes uint8 [..., K/32])."""
    exps = block_exponents(x)
    return encode(x, exps), exps


def dequantize(codes, exps) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    K = codes.shape[-1]
    vals = nvfp4.E2M1_VALUES[codes].reshape(*codes.shape[:-1], K // BLOCK, BLOCK)
    scale = np.ldexp(1.0, np.asarray(exps, dtype=np.int64) - E8M0_BIAS)[..., None]
    return (vals * scale).reshape(codes.shape)


def linear(x, w_codes, w_exps) -> np.ndarray:
    """y [M, N] = Q(x) Q(W)^T, x [M, K] quantised to MXFP4 on the fly."""
    xc, xe = quantize(x)
    return dequantize(xc, xe) @ dequantize(w_codes, w_exps).T


# --------------------------------------------------------------------------
# The mixture-of-experts layer in OCP MXFP4.
# --------------------------------------------------------------------------
# The emulation backend's OCP MX path runs the MoE experts of MXFP4 models
# (vLLM PR #35737, "Purpose": TritonExperts for OCP MX emulation).  The
# reading taken: the NVFP4 layer (oracle.moe.layer, W4A4) with MXFP4 in place
# of NVFP4 for the activations, the expert weights and the intermediate; all
# block scales are computed from the tensor itself (dynamic), and since an
# E8M0 scale spans the whole FP32 range there is no global scale and nothing
# to calibrate.


class MxExpertWeights:
    """MXFP4 expert weights, quantised on demand from FP32.

    ``src13(e)`` returns the FP32 [2I, H] gate/up weight of expert slot e and
    ``src2(e)`` the FP32 [H, I] down weight (blocks of 32 along the
    contraction dimension)."""

    def __init__(self, src13, src2):
        self._src = {13: src13, 2: src2}
        self._cache: dict = {}

    @classmethod
    def from_arrays(cls, w13, w2):
        w13 = np.asarray(w13, dtype=np.float32)
        w2 = np.asarray(w2, dtype=np.float32)
        return cls(lambda e: w13[e], lambda e: w2[e])

    def quantized(self, which: int, e: int):
        """(codes uint8 [N, K], exponent bytes uint8 [N, K/32])."""
        key = (which, int(e))
        if key not in self._cache:
            self._cache[key] = quantize(np.asarray(self._src[which](int(e)), dtype=np.float32))
        return self._cache[key]

    def dequantized(self, which: int, e: int) -> np.ndarray:
        return dequantize(*self.quantized(which, e))


def layer(x, topk_ids, topk_w, weights: MxExpertWeights, n_routed: int, I: int, shared: int = 0,
          tokens=None):
    """One MXFP4 expert layer (FP64).  Returns a dict with out [T, H], the
    alignment (offsets, sorted_pair, inv_pos), a1 codes/exponents, the sorted
    rows computed, h (pre-requantisation), a2 codes/exponents and d."""
    from . import moe
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    k = np.asarray(topk_ids).shape[1]
    offsets, sorted_pair, inv_pos = moe.align(topk_ids, n_routed, shared)
    a1c, a1e = quantize(x)
    x_hat = dequantize(a1c, a1e)
    keep = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    out = np.zeros((T, H))
    rows_all, h_all, c_all, e_all, d_all = [], [], [], [], []
    for e in range(len(offsets) - 1):
        rows = np.arange(offsets[e], offsets[e + 1])
        tok, wgt = moe.pair_token_weight(sorted_pair[rows], T, k, topk_w)
        sel = keep[tok]
        rows, tok, wgt = rows[sel], tok[sel], wgt[sel]
        if rows.size == 0:
            continue
        h = moe.swiglu(x_hat[tok] @ weights.dequantized(13, e).T, I)
        a2c, a2e = quantize(h)
        d = dequantize(a2c, a2e) @ weights.dequantized(2, e).T
        np.add.at(out, tok, wgt[:, None] * d)
        rows_all.append(rows)
        h_all.append(h)
        c_all.append(a2c)
        e_all.append(a2e)
        d_all.append(d)

    def cat(lst, width, dtype=np.float64):
        return np.concatenate(lst) if lst else np.zeros((0, width), dtype=dtype)

    return {"out": out, "offsets": offsets, "sorted_pair": sorted_pair, "inv_pos": inv_pos,
            "a1_codes": a1c, "a1_exps": a1e,
            "rows": np.concatenate(rows_all) if rows_all else np.zeros(0, dtype=np.int64),
            "h": cat(h_all, I), "a2_codes": cat(c_all, I, np.uint8).astype(np.uint8),
            "a2_exps": cat(e_all, I // BLOCK, np.uint8).astype(np.uint8), "d": cat(d_all, H)}


def down_and_combine(a2_hat, rows, sorted_pair, offsets, topk_w, weights: MxExpertWeights,
                     T: int, k: int) -> np.ndarray:
    """The layer's second half from given dequantised intermediate rows."""
    from . import moe
    rows = np.asarray(rows, dtype=np.int64)
    H = weights.dequantized(2, 0).shape[0]
    out = np.zeros((T, H))
    expert_of_row = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(expert_of_row):
        sel = expert_of_row == e
        tok, wgt = moe.pair_token_weight(sorted_pair[rows[sel]], T, k, topk_w)
        np.add.at(out, tok, wgt[:, None] * (a2_hat[sel] @ weights.dequantized(2, int(e)).T))
    return out


def near_tie_mask(x, rel: float = 2.0 ** -12, abs_tol: float = 0.0):
    """Flags (element_mask [..., K], block_mask [..., K/32]) where an input
    carrying accumulation error may legitimately round the other way: a block
    whose amax lies within rel * b + abs_tol of a power of two b (where
    floor(log2 amax), hence the exponent byte, changes), an element whose |x|
    lies that close to t * X for an E2M1 midpoint t and the block scale X."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    blocks = np.abs(x.reshape(*x.shape[:-1], K // BLOCK, BLOCK))
    amax = blocks.max(axis=-1)
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
    lo = np.ldexp(1.0, fe - 1)                     # power of two at or below amax
    hi = 2.0 * lo
    d = np.minimum(np.abs(amax - lo) - rel * lo, np.abs(hi - amax) - rel * hi)
    block_flag = (amax > 0) & (d <= abs_tol)
    X = np.ldexp(1.0, block_exponents(x).astype(np.int64) - E8M0_BIAS)[..., None, None]
    b2 = X * nvfp4._midpoints(nvfp4.E2M1_MAGS)     # [..., K/32, 1, 7]
    de = np.min(np.abs(blocks[..., None] - b2) - rel * b2, axis=-1)
    elem_flag = (de <= abs_tol).reshape(x.shape)
    return elem_flag, block_flag
