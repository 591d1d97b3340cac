// Per-lane NVFP4 block quantisation shared by the quantisation kernels.
//
// A lane takes one 16-element block of a row, so the block amax, the scale
// decision and the bounds of the code decisions are computed once per block
// (with a lane per 8 elements both lanes of a block repeated them; measured
// on the large-batch fused path: prefill W4A4 388 -> 386 us, skew 733 -> 727
// us).  Decisions are exact (see common.h): the E4M3 block scale is the
// nearest value to amax / (6 g), the E2M1 codes the nearest magnitudes to
// |x| / (s g), ties to the even code.
#pragma once

#include "common.h"

namespace nvfp4 {

// Load 8 consecutive elements as floats (x is 16-byte aligned at i).
__device__ __forceinline__ void load8(const uint16_t* x, int64_t i, float v[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(x + i);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
  }
}
__device__ __forceinline__ void load8(const float* x, int64_t i, float v[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(x + i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(x + i + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = b[j];
  }
}

// Cross-workgroup step of a global scale: workgroup maxima are folded into
// ws_max (float bits of a non-negative value order like unsigned integers)
// and counted in ws_cnt; the last of nblk workgroups writes g and puts both
// words back to zero, so the workspace is ready for the next call (it must be
// zero before the first one).
//
// Both words are only ever touched by device-scope atomics, which every
// workgroup performs at the same place, and the count is issued only after
// the fetch-max has returned (the count's operand depends on its result), so
// the workgroup that counts last reads the complete maximum.  No workgroup
// wrote plain data that another reads, so no release/acquire fence is taken:
// at device scope those write back and invalidate the XCD's L2, and a
// thousand of them serialised on one counter cost tens of microseconds.
__device__ __forceinline__ void fold_max_and_count(uint32_t* ws_cnt, uint32_t* ws_max, float m,
                                                   uint32_t nblk, float* g) {
  const uint32_t old = __hip_atomic_fetch_max(ws_max, (uint32_t)__float_as_int(m), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  // old < 2^31 (bits of a non-negative float), so the increment is 1, but it
  // cannot be issued before the fetch-max has completed.
  const uint32_t done = __hip_atomic_fetch_add(ws_cnt, 1u + (old >> 31), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
  if (done == nblk - 1) {
    const uint32_t bits = __hip_atomic_fetch_max(ws_max, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *g = global_scale_of_amax(__int_as_float((int)bits));
    __hip_atomic_store(ws_max, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ws_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One 16-byte load as floats: 8 bf16 or 4 FP32 elements (x + i 16-byte aligned).
__device__ __forceinline__ void load_vec(const uint16_t* x, int64_t i, float (&v)[8]) { load8(x, i, v); }
__device__ __forceinline__ void load_vec(const float* x, int64_t i, float (&v)[4]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(x + i);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = a[j];
}

// Quantise the 16 values v of elements [c16, c16 + 16) of row ``row`` (one
// block, one lane: the scale decision is taken once per block).  Writes the
// 16 codes (8 bytes), the block scale and, with x_deq, the exact f16 values
// code * scale.
__device__ __forceinline__ void quantize_block_values(const float (&v)[16], int64_t row, int64_t c16, int64_t K,
                                                      float gv, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ sf, uint16_t* __restrict__ x_deq) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, amax_input(v[j]));
  const uint32_t sc = e4m3_scale_code(m, gv);
  const float s = e4m3_value(sc);
  const E2M1Bounds bd = e2m1_bounds(s, gv);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w0 |= e2m1_code(v[j], bd, sc == 0) << (4 * j);
    w1 |= e2m1_code(v[8 + j], bd, sc == 0) << (4 * j);
  }
  *reinterpret_cast<u32x2*>(q + row * (K >> 1) + (c16 >> 1)) = u32x2{w0, w1};
  sf[row * (K >> 4) + (c16 >> 4)] = (uint8_t)sc;
  // The exact f16 values code * scale (at most six significant bits, in
  // [2^-10, 2688]): the hardware FP4 convert, then one packed multiply by the
  // scale per pair.
  if (x_deq) {
    const f16x2 s2 = f16x2_splat(s);
    *reinterpret_cast<f16x8*>(x_deq + row * K + c16) = dequant8_f16(w0, s2);
    *reinterpret_cast<f16x8*>(x_deq + row * K + c16 + 8) = dequant8_f16(w1, s2);
  }
}

// The same, loading the 16 elements from x (16-byte aligned at row * ldx + c16).
template <typename T>
__device__ __forceinline__ void quantize_block(const T* __restrict__ x, int64_t row, int64_t c16, int64_t K,
                                               int64_t ldx, float gv, uint8_t* __restrict__ q,
                                               uint8_t* __restrict__ sf, uint16_t* __restrict__ x_deq) {
  float v[16];
  load8(x, row * ldx + c16, *reinterpret_cast<float (*)[8]>(&v[0]));
  load8(x, row * ldx + c16 + 8, *reinterpret_cast<float (*)[8]>(&v[8]));
  quantize_block_values(v, row, c16, K, gv, q, sf, x_deq);
}

// Half a block per lane (8 elements; the two lanes of a block are adjacent,
// even lane first, and share the block amax by one DPP exchange): for
// decode-sized tensors, where the lanes of the fused kernel outnumber the
// blocks and a shorter chain per lane matters more than the repeated scale
// decision.  Same decisions and outputs as quantize_block_values.
__device__ __forceinline__ void quantize_half_block_values(const float (&v)[8], int64_t row, int64_t c8,
                                                           int64_t K, float gv, uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ sf,
                                                           uint16_t* __restrict__ x_deq) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, amax_input(v[j]));
  m = fmaxf(m, dpp_xor1(m));
  const uint32_t sc = e4m3_scale_code(m, gv);
  const float s = e4m3_value(sc);
  const E2M1Bounds bd = e2m1_bounds(s, gv);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) word |= e2m1_code(v[j], bd, sc == 0) << (4 * j);
  *reinterpret_cast<uint32_t*>(q + row * (K >> 1) + (c8 >> 1)) = word;
  if ((c8 & 15) == 0) sf[row * (K >> 4) + (c8 >> 4)] = (uint8_t)sc;
  if (x_deq) *reinterpret_cast<f16x8*>(x_deq + row * K + c8) = dequant8_f16(word, f16x2_splat(s));
}

// OCP MXFP4 encoding of 8 consecutive elements of a row by one lane; the
// four lanes of a 32-element block are a DPP quad (the block maximum is two
// exchanges), so all four must call this together.  Returns the 8 codes
// (element j in nibble j) and sets ebyte to the block's E8M0 byte:
// floor(log2 amax) - 2 + 127 clamped to [0, 254] (0 for an all-zero block);
// each code is the nearest E2M1 value to v / 2^(ebyte - 127), ties to the
// even code, above 6 saturating, the sign kept.
__device__ __forceinline__ uint32_t mx_encode8(const float (&v)[8], int& ebyte) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, amax_input(v[j]));
  m = fmaxf(m, dpp_xor1(m));
  m = fmaxf(m, dpp_xor2(m));
  // floor(log2 m) = frexp exponent - 1 (m = f * 2^E, f in [0.5, 1)).
  ebyte = m > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(m) - 1 - 2 + 127, 0), 254) : 0;
  const int sh = 127 - ebyte;   // v / scale = v * 2^sh, exact
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = fabsf(__builtin_ldexpf(v[j], sh));
    // nearest of {0,.5,1,1.5,2,3,4,6}; ties to the even code (up at .75,
    // 1.75, 3.5; down at .25, 1.25, 2.5, 5); above 6 saturates
    const uint32_t mag = (uint32_t)(a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                         (a >= 3.5f) + (a > 5.0f);
    const uint32_t sign = ((uint32_t)__float_as_int(v[j]) >> 28) & 8u;
    word |= (sign | mag) << (4 * j);
  }
  return word;
}

// The same with the canonical stores: q [rows][K/2] gets the 8 codes, ex
// [rows][K/32] the exponent byte (from the first lane of the block).
__device__ __forceinline__ void mx_quantize8_canonical(const float (&v)[8], int64_t row, int64_t c8, int64_t K,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ ex) {
  int ebyte;
  const uint32_t word = mx_encode8(v, ebyte);
  *reinterpret_cast<uint32_t*>(q + row * (K >> 1) + (c8 >> 1)) = word;
  if ((c8 & 31) == 0) ex[row * (K >> 5) + (c8 >> 5)] = (uint8_t)ebyte;
}

}  // namespace nvfp4
