"""Token-by-token dense recomputation of the expert layer (test infrastructure).

FlashInfer #2723 ("The Problem") found a grouped block-scaled GEMM producing
garbage while the dense FP4 GEMM was right.  This module therefore restates the
layer without any grouping, permutation or batching: for each token, for each
of its experts, one dense matrix-vector product per projection, accumulated in
FP64 in the order of the token's expert list.  ``tests`` compare it with the
grouped ``oracle.moe.layer`` on small workloads.  The activation comes from
torch (``torch.nn.functional.silu`` in FP64), not from ``oracle.moe``, so a
mistake in either implementation of the SwiGLU step shows as a mismatch.
"""
from __future__ import annotations

import numpy as np
import torch

from . import nvfp4


def _silu(z):
    """silu through torch's own FP64 CPU kernel (z * sigmoid(z)), a second,
    independent implementation of the activation next to ``moe.silu``."""
    return torch.nn.functional.silu(torch.from_numpy(np.asarray(z, dtype=np.float64))).numpy()


def layer_per_token(x, topk_ids, topk_w, w13_hat, w2_hat, I: int, variant: str = "w4a4",
                    g2=None, shared_w13=None, shared_w2=None) -> np.ndarray:
    """Dense per-token loop.  ``w13_hat``/``w2_hat`` are FP64 dequantised
    weights [E, 2I, H] / [E, H, I]; the optional shared expert is given
    separately and added with weight 1."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_w, dtype=np.float64)
    if variant == "w4a4":
        g1 = nvfp4.global_scale(x)
        x_hat = nvfp4.dequantize(*nvfp4.quantize(x, g1), g1)
    else:
        x_hat = x
    out = np.zeros((T, H))

    def mlp(xv, W13, W2):
        gate = np.array([np.dot(W13[i], xv) for i in range(I)])
        up = np.array([np.dot(W13[I + i], xv) for i in range(I)])
        h = _silu(gate) * up
        if variant == "w4a4":
            h = nvfp4.dequantize(*nvfp4.quantize(h[None, :], g2), g2)[0]
        else:
            h = nvfp4.round_to_bf16(h)
        return np.array([np.dot(W2[r], h) for r in range(H)])

    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            out[t] += wts[t, j] * mlp(x_hat[t], w13_hat[e], w2_hat[e])
        if shared_w13 is not None:
            out[t] += mlp(x_hat[t], shared_w13, shared_w2)
    return out


def mx_layer_per_token(x, topk_ids, topk_w, w13_hat, w2_hat, I: int, shared_w13=None,
                       shared_w2=None) -> np.ndarray:
    """The OCP MXFP4 layer token by token (dense products, FP64, the token's
    experts in list order); the activation and intermediate are MXFP4
    quantise-dequantised per token row."""
    from . import mxfp4
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_w, dtype=np.float64)
    x_hat = mxfp4.dequantize(*mxfp4.quantize(x))
    out = np.zeros((T, H))

    def mlp(xv, W13, W2):
        gate = np.array([np.dot(W13[i], xv) for i in range(I)])
        up = np.array([np.dot(W13[I + i], xv) for i in range(I)])
        h = _silu(gate) * up
        h = mxfp4.dequantize(*mxfp4.quantize(h[None, :]))[0]
        return np.array([np.dot(W2[r], h) for r in range(H)])

    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            out[t] += wts[t, j] * mlp(x_hat[t], w13_hat[e], w2_hat[e])
        if shared_w13 is not None:
            out[t] += mlp(x_hat[t], shared_w13, shared_w2)
    return out
