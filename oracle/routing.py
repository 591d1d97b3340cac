"""Router reference: softmax, top-k, renormalise (test infrastructure only).

The mixture-of-experts layers on the pages route each token to its top-k
experts ("512 routed + 1 shared, 10 routed per token", FlashInfer #2723,
"Model" table).  The pages do not spell out the router; the reading taken here
is the usual one: take the k largest logits (ties to the lower expert id) and
weight them by the softmax over all experts renormalised over the k chosen
ones.  Because the softmax denominator cancels in the renormalisation, the
weights equal the softmax over the k chosen logits alone; ``route_topk`` uses
that closed form and the tests check it against the two-step definition.
"""
from __future__ import annotations

import numpy as np


def route_topk(logits, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Return (ids int32 [T, k], weights float32 [T, k]).

    ``logits`` is FP32 [T, E].  Experts are ordered by decreasing logit, equal
    logits by increasing id.  Weights are computed in FP64 and rounded to FP32.
    """
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-z, axis=1, kind="stable")      # stable: lower id first on ties
    ids = order[:, :k]
    w = selected_weights_f64(np.take_along_axis(z, ids, axis=1))
    return ids.astype(np.int32), w.astype(np.float32)


def selected_weights_f64(sel) -> np.ndarray:
    """FP64 softmax over the selected logits [T, k] (column 0 the largest):
    exp(z_j - z_0) / sum_i exp(z_i - z_0), the sum taken in the order
    i = 0, 1, ..., k-1 (the order fixes the FP64 rounding of the sum)."""
    sel = np.asarray(sel, dtype=np.float64)
    ex = np.exp(sel - sel[:, :1])
    s = ex[:, 0].copy()
    for j in range(1, ex.shape[1]):
        s = s + ex[:, j]
    return ex / s[:, None]


def fp32_rounding_near_tie(v, rel: float = 2.0 ** -40) -> np.ndarray:
    """True where the FP64 value v lies within ``rel`` (relative) of a point
    halfway between two neighbouring FP32 numbers: there, an FP64 result that
    differs from this one by a few FP64 ulps (another exp implementation) may
    round to the other FP32 neighbour.  For normal FP32 magnitudes only."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= m < 1
    ulp = np.ldexp(1.0, e - 24)              # FP32 spacing at v
    lo = np.floor(v / ulp) * ulp             # FP32 neighbour below (exact)
    mid = lo + 0.5 * ulp
    return (v > 0) & (np.abs(v - mid) <= rel * v)


def route_two_step(logits, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Definition form: full softmax, pick top-k, divide by their sum (FP64)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    ids = np.argsort(-z, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(p, ids, axis=1)
    return ids.astype(np.int32), (sel / sel.sum(axis=1, keepdims=True))
