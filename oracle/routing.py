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
    sel = np.take_along_axis(z, ids, axis=1)
    ex = np.exp(sel - sel[:, :1])                      # sel[:, 0] is the row maximum
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def route_two_step(logits, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Definition form: full softmax, pick top-k, divide by their sum (FP64)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    ids = np.argsort(-z, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(p, ids, axis=1)
    return ids.astype(np.int32), (sel / sel.sum(axis=1, keepdims=True))
