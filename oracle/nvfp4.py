"""NVFP4 block format, FP64 reference (test infrastructure only).

What the pages fix about the format:

* Values are 4-bit E2M1 floats with an FP8 block scale ("FP4 weights with FP8
  block scales", FlashInfer #2723, "Model" table).
* The block scale is an unsigned E4M3 number and one scale covers 16 elements
  along the contraction dimension: the native instruction named in unsloth PR
  #10417 ("Why it matters") multiplies E2M1 by E2M1 with UE4M3 scales, four
  scales per 64-deep step.
* Per-block amax and the scale are computed in FP32 (FlashInfer #2723, "2. FP32
  Amax Computation").
* Activations are quantised from BF16 on the fly, per token (FlashInfer #2723,
  "Why 39 vs 49 tok/s?").

Readings where the pages are silent (each one is also listed in the design doc):

* E2M1 is sign | 2 exponent bits | 1 mantissa bit, exponent bias 1, so the
  magnitudes of codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 are the
  same magnitudes with the sign bit set.
* E4M3 is the OCP "FN" variant: bias 7, no infinities, 0x7F is NaN, largest
  finite 448, subnormals m * 2^-9.  Scale bytes have the sign bit clear.
* A tensor (activations) or an expert matrix (weights) has one FP32 global
  scale g = fl32(amax / (6 * 448)): 6 is the largest E2M1 magnitude and 448 the
  largest E4M3 value, so the largest block scale lands at the top of E4M3.
* Decoding: value = (-1)^sign * E2M1[code] * E4M3[scale] * g.
* Encoding a 16-element block with global scale g:
    s = round_E4M3(amax_block / (6 g)),  saturating at 448;
    code_i = sign(x_i) | round_E2M1(|x_i| / (s g)),  saturating at 6.
  Both roundings are to nearest on the exact real quotient, ties to the even
  code.  A block whose scale rounds to 0 gets magnitude code 0 everywhere.
  The sign bit is the IEEE sign of the input, so -0.0 and negative values that
  round to zero encode as 0x8.
* Packing: byte j of a row holds element 2j in its low nibble and element
  2j+1 in its high nibble; scales are one byte per block, row-major.

Exactness: the inputs here are BF16 or FP32 (at most 24 significant bits) and g
is FP32.  The rounding thresholds, 6*g*m for an E4M3 midpoint m and t*s*g for
an E2M1 midpoint t, have at most 31 significant bits, so they are exact FP64
numbers.  An input equal to a threshold is therefore detected exactly, and an
input that differs from one differs by at least 2^-32 of its value; an FP64
quotient (relative error 2^-53) thus lands on the same side of every midpoint
as the real quotient.  Every decision below is the exact-real decision.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# Code tables, built from the bit-field definitions.
# --------------------------------------------------------------------------
def e2m1_magnitude(code: int) -> float:
    """Magnitude of a 3-bit E2M1 code (exponent bits e, mantissa bit m, bias 1)."""
    e, m = (code >> 1) & 3, code & 1
    if e == 0:                       # subnormal: m * 2^(1 - bias) * 2^-1
        return 0.5 * m
    return (1.0 + 0.5 * m) * 2.0 ** (e - 1)


def e2m1_value(code: int) -> float:
    """Signed value of a 4-bit E2M1 code."""
    v = e2m1_magnitude(code & 7)
    return -v if code & 8 else v


def e4m3_value(code: int) -> float:
    """Value of an 8-bit OCP E4M3 (FN) code: bias 7, no infinities."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:                       # subnormal: m/8 * 2^(1 - bias)
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E2M1_MAGS = np.array([e2m1_magnitude(c) for c in range(8)], dtype=np.float64)
E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
# Non-negative finite E4M3 values, indexed by code 0x00..0x7E (ascending).
E4M3_POS = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)


# --------------------------------------------------------------------------
# Round to nearest, ties to even code, on exact quotients.
# --------------------------------------------------------------------------
def _midpoints(grid: np.ndarray) -> np.ndarray:
    return (grid[:-1] + grid[1:]) / 2.0            # exact: few significant bits


def round_quotient_to_grid(num: np.ndarray, den: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index c into ascending ``grid`` nearest to the real number num/den.

    ``num >= 0`` and ``den > 0`` are FP64 arrays (broadcast together).  The
    midpoint between grid[c] and grid[c+1] is crossed when num > den*mid, or
    when num == den*mid and c+1 is even (ties to the even code).  Values above
    the last midpoint take the last index (saturation).  The caller guarantees
    that den*mid is exact in FP64.
    """
    num = np.asarray(num, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    mids = _midpoints(grid)
    upper_is_even = (np.arange(1, len(grid)) % 2) == 0
    if den.ndim == 0 and len(grid) <= 16:
        # Few midpoints: count the crossed ones directly.
        out = np.zeros(num.shape, dtype=np.int64)
        for m, up in zip(float(den) * mids, upper_is_even):
            out += (num > m) | ((num == m) & up)
        return out
    if den.ndim == 0:
        # One denominator for all: the thresholds den*mid form one sorted list.
        thr = float(den) * mids
        crossed = np.searchsorted(thr, num, side="left")      # #{mid : num > den*mid}
        at = np.minimum(crossed, len(thr) - 1)
        tie = (crossed < len(thr)) & (num == thr[at]) & upper_is_even[at]
        return crossed + tie
    num_b, den_b = np.broadcast_arrays(num, den)
    out = np.zeros(num_b.shape, dtype=np.int64)
    flat_n, flat_d, flat_o = num_b.reshape(-1), den_b.reshape(-1), out.reshape(-1)
    step = 1 << 16
    for s in range(0, flat_n.size, step):
        n = flat_n[s:s + step, None]
        thr = flat_d[s:s + step, None] * mids[None, :]
        flat_o[s:s + step] = (n > thr).sum(1) + ((n == thr) & upper_is_even[None, :]).sum(1)
    return out


# --------------------------------------------------------------------------
# Global scale.
# --------------------------------------------------------------------------
def global_scale(x) -> np.float32:
    """g = fl32(max|x| / 2688) for a whole tensor (or expert matrix).

    The FP64 quotient rounded to FP32 equals the correctly rounded FP32
    quotient (53 >= 2*24 + 2 bits, so the double rounding is innocuous).
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    amax = float(a.max()) if a.size else 0.0
    return np.float32(amax / (E2M1_MAX * E4M3_MAX))


# --------------------------------------------------------------------------
# Quantise / dequantise.
# --------------------------------------------------------------------------
def block_scales(x, g) -> np.ndarray:
    """E4M3 scale codes uint8 [..., K/16]: nearest E4M3 value to amax/(6 g)."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("contraction length must be a multiple of 16")
    g = float(np.float32(g))
    amax = np.abs(x.reshape(*x.shape[:-1], K // BLOCK, BLOCK)).max(axis=-1)
    scale_code = round_quotient_to_grid(amax, np.float64(E2M1_MAX * g), E4M3_POS)
    return np.where(amax == 0.0, 0, scale_code).astype(np.uint8)


def encode_with_scales(x, scales, g) -> np.ndarray:
    """E2M1 codes uint8 [..., K] of x given its block scale codes."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    g = float(np.float32(g))
    blocks = x.reshape(*x.shape[:-1], K // BLOCK, BLOCK)
    mag = np.abs(blocks)
    s_val = E4M3_POS[np.asarray(scales, dtype=np.int64)]
    # Element magnitudes: nearest E2M1 magnitude to r = |x| / (s g).  The FP64
    # quotient is exact when r is an E2M1 midpoint and otherwise stays on the
    # same side of every midpoint (see the module note), so rounding it
    # decides as the real quotient would.
    den = (s_val * g)[..., None]
    r = mag / np.where(den > 0.0, den, 1.0)
    mag_code = round_quotient_to_grid(r, np.float64(1.0), E2M1_MAGS)
    mag_code = np.where((s_val[..., None] == 0.0) | (mag == 0.0), 0, mag_code)
    sign = np.signbit(blocks).astype(np.int64)
    return (mag_code | (sign << 3)).reshape(x.shape).astype(np.uint8)


def quantize(x, g) -> tuple[np.ndarray, np.ndarray]:
    """Encode ``x`` [..., K] (K % 16 == 0) with global scale ``g``.

    Returns (codes uint8 [..., K] with values 0..15, scales uint8 [..., K/16]).
    """
    scales = block_scales(x, g)
    return encode_with_scales(x, scales, g), scales


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """FP64 values code * scale * g (exact)."""
    codes = np.asarray(codes, dtype=np.int64)
    K = codes.shape[-1]
    vals = E2M1_VALUES[codes].reshape(*codes.shape[:-1], K // BLOCK, BLOCK)
    s = E4M3_POS[np.asarray(scales, dtype=np.int64)][..., None]
    return (vals * s * float(np.float32(g))).reshape(codes.shape)


def quantize_packed(x, g) -> tuple[np.ndarray, np.ndarray]:
    """Quantise and pack: (bytes uint8 [..., K/2], scales uint8 [..., K/16])."""
    codes, scales = quantize(x, g)
    return pack_codes(codes), scales


def dequantize_packed(packed, scales, g) -> np.ndarray:
    return dequantize(unpack_codes(packed), scales, g)


# --------------------------------------------------------------------------
# Near ties: where an FP32-accumulated input may legitimately round the other
# way.  Used to judge the requantised intermediate of the expert layer.
# --------------------------------------------------------------------------
def near_tie_mask(x, g, rel: float = 2.0 ** -12, abs_tol: float = 0.0) -> tuple[np.ndarray, np.ndarray]:
    """Flags (element_mask [..., K], block_mask [..., K/16]).

    A block is flagged when amax lies within ``rel`` (relative) plus
    ``abs_tol`` (absolute, in units of x) of a value 6*g*m at which its E4M3
    scale would round differently; an element is flagged when |x| lies that
    close to a value t*s*g at which its E2M1 code would.  Used to judge an
    input computed with accumulation error: both roundings are correct there.
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    g = float(np.float32(g))
    blocks = np.abs(x.reshape(*x.shape[:-1], K // BLOCK, BLOCK))
    amax = blocks.max(axis=-1)
    b4 = 6.0 * g * _midpoints(E4M3_POS)
    d = np.min(np.abs(amax[..., None] - b4) - rel * b4, axis=-1)
    block_flag = d <= abs_tol
    sc = block_scales(x, g)
    sg = (E4M3_POS[sc.astype(np.int64)] * g)[..., None, None]
    b2 = sg * _midpoints(E2M1_MAGS)                    # [..., K/16, 1, 7]
    de = np.min(np.abs(blocks[..., None] - b2) - rel * b2, axis=-1)
    elem_flag = ((de <= abs_tol) & (sg[..., 0] > 0)).reshape(x.shape)
    return elem_flag, block_flag


# --------------------------------------------------------------------------
# bfloat16 rounding (the W4A16 intermediate).
# --------------------------------------------------------------------------
def round_to_bf16(v) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits), ties to even, as FP64."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                        # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                   # below 2^-126 the quantum is fixed
    q = np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)
    return np.where(v == 0.0, v, q)
