"""Dense NVFP4 linear layer reference: y = x W^T (FP64 NumPy).

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and
bench.py's CPU baseline, never by the product path.

The pages' second workload besides the expert layer is the plain NVFP4
linear layer, timed per GEMM across batch sizes M with NVFP4 activations
(W4A4) against bf16 activations and in-kernel weight dequantisation (W4A16)
(unsloth PR #10417, "Why it matters" and its kernel-selection results).
What is computed follows the expert path's conventions (see oracle/moe.py):

* W4A4: the activations get a dynamic global scale g = fl32(max|x| / 2688)
  and block quantisation (oracle/nvfp4.py); the result is the FP64 product of
  the dequantised activations and dequantised weights, i.e. the FP32
  accumulator times alpha = g * gw taken exactly.
* W4A16: bf16 activations times the dequantised weights.
"""
from __future__ import annotations

import numpy as np

from . import nvfp4


def quantize_weight(w):
    """(codes uint8 [N, K], scales uint8 [N, K/16], gw float32) of FP32 w [N, K]."""
    w = np.asarray(w, dtype=np.float32)
    gw = nvfp4.global_scale(w)
    codes, scales = nvfp4.quantize(w, gw)
    return codes, scales, gw


def linear_w4a4(x, w_codes, w_scales, gw) -> np.ndarray:
    """y [M, N] = Q(x) Q(W)^T with x [M, K] (bf16 values) quantised on the fly."""
    x = np.asarray(x, dtype=np.float64)
    g = nvfp4.global_scale(x)
    codes, scales = nvfp4.quantize(x, g)
    x_hat = nvfp4.dequantize(codes, scales, g)
    w_hat = nvfp4.dequantize(w_codes, w_scales, gw)
    return x_hat @ w_hat.T


def linear_w4a16(x, w_codes, w_scales, gw) -> np.ndarray:
    """y [M, N] = x Q(W)^T with x [M, K] used as given (bf16 values, exact in FP64)."""
    x = np.asarray(x, dtype=np.float64)
    w_hat = nvfp4.dequantize(w_codes, w_scales, gw)
    return x @ w_hat.T
