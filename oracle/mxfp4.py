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
