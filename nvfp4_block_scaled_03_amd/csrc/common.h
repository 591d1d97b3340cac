// Device helpers shared by the NVFP4 MoE kernels (gfx950 only).
//
// Format facts (see include/nvfp4_moe.h for the pages they come from): E2M1
// element codes, one unsigned E4M3 block scale per 16 elements along the
// contraction dimension, one FP32 global scale per tensor or expert matrix.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Cross-lane helpers (DPP within rows of 16 lanes).
// ---------------------------------------------------------------------------
// quad_perm [1,0,3,2]: exchange with lane ^ 1.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ int dpp_xor1_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
}
// quad_perm [2,3,0,1]: exchange with lane ^ 2.
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// row_half_mirror: lane i <-> 7 - i within each half-row of 8.
__device__ __forceinline__ float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}
// row_mirror: lane i <-> 15 - i within each row of 16.
__device__ __forceinline__ float dpp_row_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
}
// Maximum over the 16 lanes of a DPP row (every lane gets the result).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, dpp_half_mirror(v));
  v = fmaxf(v, dpp_row_mirror(v));
  return v;
}

// ---------------------------------------------------------------------------
// Exact rounding decisions.
//
// Block scale: s = nearest E4M3 value to q = amax / (6 g), ties to the even
// code, saturating at 448.  6*g is exact in FP64 and the FP64 quotient is
// correctly rounded; amax (24 significant bits) and 6*g*m for an E4M3
// midpoint m (at most 31 bits) are either equal or differ by at least 2^-32
// relative, far above the 2^-53 rounding of the quotient, so rounding the
// FP64 quotient decides exactly as the real quotient would.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax, float g) {
  if (!(amax > 0.0f)) return 0u;
  const double q = (double)amax / (6.0 * (double)g);
  if (!(q < 448.0)) return 0x7Eu;                       // saturate (also g == 0)
  if (q < 0.015625) return (uint32_t)__builtin_rint(q * 512.0);   // subnormal step 2^-9
  int e2;
  (void)__builtin_frexp(q, &e2);                         // q = m * 2^e2, m in [0.5, 1)
  const int e = e2 - 1;                                  // q in [2^e, 2^(e+1)), e in [-6, 8]
  const double r = __builtin_rint(__builtin_ldexp(q, 3 - e));  // in [8, 16]
  return (uint32_t)((e + 6) * 8 + (int)r);
}

// Value of a non-negative E4M3 code 0x00..0x7E.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;            // m * 2^-9
  return __int_as_float((int)(((e + 120u) << 23) | (m << 20)));  // (1 + m/8) * 2^(e-7)
}

// Largest float <= d (d > 0).
__device__ __forceinline__ float f32_round_down(double d) {
  float f = (float)d;
  if ((double)f > d) f = __int_as_float(__float_as_int(f) - 1);
  return f;
}
// Largest float strictly below the smallest float >= d (d > 0): comparing
// v > result is the same as v >= d for every float v.
__device__ __forceinline__ float f32_below_round_up(double d) {
  float f = (float)d;
  if ((double)f < d) f = __int_as_float(__float_as_int(f) + 1);
  return __int_as_float(__float_as_int(f) - 1);
}

// The seven decision boundaries between consecutive E2M1 magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} for block scale s and global scale g, as
// floats c[i] such that  magnitude code = #{ i : |x| > c[i] }.
// The real boundaries are t_i * s * g with t = .25 .75 1.25 1.75 2.5 3.5 5;
// they have at most 31 significant bits, so they are exact in FP64.  A tie
// goes to the even code: up at .75, 1.75, 3.5 and down at the others.
struct E2M1Bounds {
  float c0, c1, c2, c3, c4, c5, c6;
};
__device__ __forceinline__ E2M1Bounds e2m1_bounds(float s, float g) {
  const double t = (double)s * (double)g;
  E2M1Bounds b;
  b.c0 = f32_round_down(0.25 * t);
  b.c1 = f32_below_round_up(0.75 * t);
  b.c2 = f32_round_down(1.25 * t);
  b.c3 = f32_below_round_up(1.75 * t);
  b.c4 = f32_round_down(2.5 * t);
  b.c5 = f32_below_round_up(3.5 * t);
  b.c6 = f32_round_down(5.0 * t);
  return b;
}
// Magnitude code (0..7) of |x| by a three-level search over the bounds.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a, const E2M1Bounds& b) {
  const bool hi = a > b.c3;
  const float m1 = hi ? b.c5 : b.c1;
  const bool mid = a > m1;
  const float m0 = hi ? (mid ? b.c6 : b.c4) : (mid ? b.c2 : b.c0);
  const bool lo = a > m0;
  return ((uint32_t)hi << 2) | ((uint32_t)mid << 1) | (uint32_t)lo;
}
// Full 4-bit code of x (sign from the IEEE sign bit; s == 0 -> magnitude 0).
__device__ __forceinline__ uint32_t e2m1_code(float x, const E2M1Bounds& b, bool zero_scale) {
  const uint32_t sign = ((uint32_t)__float_as_int(x) >> 28) & 8u;
  const uint32_t mag = zero_scale ? 0u : e2m1_mag_code(fabsf(x), b);
  return sign | mag;
}

// ---------------------------------------------------------------------------
// Dequantisation of 8 E2M1 codes (one 32-bit word, element i in nibble i)
// to exact f16 / bf16 values code * s.  The hardware FP4 convert applies
// only the exponent of its f32 scale, so it runs with scale 1.0 and the
// E4M3 scale (four significant bits) is applied with an exact multiply: the
// products have at most six significant bits and lie in [2^-10, 2688].
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 s2) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  const f16x2 q0 = p0 * s2, q1 = p1 * s2, q2 = p2 * s2, q3 = p3 * s2;
  f16x8 r;
  r[0] = q0[0]; r[1] = q0[1]; r[2] = q1[0]; r[3] = q1[1];
  r[4] = q2[0]; r[5] = q2[1]; r[6] = q3[0]; r[7] = q3[1];
  return r;
}

// bf16 version: code pairs converted to FP32 with scale 1.0, multiplied by
// s in FP32 (exact), then narrowed pairwise to bf16 (exact: six significant
// bits at most).  gfx950 has no packed bf16 multiply; this is the shortest
// exact sequence (4 instructions per pair).
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t w, float s) {
  bf16x8 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2 v = b == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
                    : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
                    : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                             : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    r[2 * b] = (__bf16)(v[0] * s);
    r[2 * b + 1] = (__bf16)(v[1] * s);
  }
  return r;
}

// Two E4M3 scale bytes (bits 0-7 and 8-15 of v) as exact f16 values {s0, s1}:
// one hardware FP8-to-f16 pair conversion (scale 1.0; exact for every E4M3
// code, verified on gfx950 for all 256 bytes).
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
}
__device__ __forceinline__ f16x2 f16x2_lo(f16x2 v) { return __builtin_shufflevector(v, v, 0, 0); }
__device__ __forceinline__ f16x2 f16x2_hi(f16x2 v) { return __builtin_shufflevector(v, v, 1, 1); }

__device__ __forceinline__ f16x2 f16x2_splat(float s) {
  const _Float16 h = (_Float16)s;
  f16x2 r;
  r[0] = h;
  r[1] = h;
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __int_as_float((int)(b << 16)); }

// Round-to-nearest-even narrowing of a finite float to bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = (uint32_t)__float_as_int(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Global scale g = fl32(amax / 2688): FP64 division then one rounding to FP32
// (53 >= 2 * 24 + 2 makes the double rounding innocuous).
__device__ __forceinline__ float global_scale_of_amax(float amax) {
  return (float)((double)amax / 2688.0);
}

// Token of pair f: routed pairs are f = t*topk + j, shared pairs f = T*topk + t.
__device__ __forceinline__ int pair_token(int f, int T, int topk) {
  const int tk = T * topk;
  return f < tk ? f / topk : f - tk;
}

}  // namespace nvfp4
