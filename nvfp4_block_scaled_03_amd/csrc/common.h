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
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
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
// Every decision compares a float |x| (or a block amax) with a real
// threshold g * M, where g is the FP32 global scale and M a small constant of
// at most 7 significant bits (6 * an E4M3 midpoint, or t * s for an E2M1
// boundary t and an E4M3 scale s).
//  - Block scale: fma(-g, M, a) rounds the exact a - g M once, and a
//    correctly rounded value has the sign of the exact one (it is zero only
//    when the exact value is, as a - g M is a multiple of a far larger power
//    of two than the smallest subnormal), so its sign is the decision.
//  - E2M1 bounds: the product g * M is split exactly into p + e with one FMA
//    (p = fl(g M), e = g M - p), which gives the floats just below and above
//    the real boundary.
// For an extremely small g (below 2^-80, where the split may underflow) both
// sides are first multiplied by 2^64, which is exact and changes no decision.
// (An earlier form took sign((a - p) - e); the compiler's contraction of
// a - g*M into an FMA made it return "equal" when g M lies exactly halfway
// between two floats.  The one-FMA form leaves nothing to contract.)
// ---------------------------------------------------------------------------

// Value of a non-negative E4M3 code 0x00..0x7E.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * 0.001953125f;                            // m * 2^-9
  const float nrm = __int_as_float((int)(((e + 120u) << 23) | (m << 20)));  // (1 + m/8) * 2^(e-7)
  return e == 0 ? sub : nrm;
}

// sign(a - g * M) for a >= 0, g > 0, M > 0 (see above).
__device__ __forceinline__ int cmp_scaled(float a, float g, float M) {
  const float d = __builtin_fmaf(-g, M, a);
  return (d > 0.0f) - (d < 0.0f);
}

// |v| as an input to a maximum that must ignore NaN.  In IEEE mode the
// hardware maximum returns the other operand for a quiet NaN but a quiet NaN
// for a signalling one, which would drop the maximum gathered so far; the
// input is therefore quietened first (canonicalisation), so any NaN, quiet or
// signalling, takes no part in the maximum.
__device__ __forceinline__ float amax_input(float v) { return fabsf(__builtin_canonicalizef(v)); }

constexpr float kTinyG = 8.271806125530277e-25f;  // 2^-80
constexpr float kLift = 18446744073709551616.0f;    // 2^64

// Block scale: s = nearest E4M3 value to q = amax / (6 g), ties to the even
// code, saturating at 448.  A candidate code comes from an approximate FP32
// quotient (within a few ulps, so at most one code off); exact checks
// against the midpoints to its two neighbours settle it.  For g < 2^-80
// both amax and g are first multiplied by 2^64, which is exact and leaves
// every decision unchanged.
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax, float g) {
  if (!(amax > 0.0f)) return 0u;
  if (g < kTinyG) {
    amax *= kLift;
    g *= kLift;
  }
  const float q = amax * __builtin_amdgcn_rcpf(6.0f * g);
  int c;
  if (!(q < 464.0f)) {
    c = 0x7E;
  } else if (q < 0.015625f) {
    c = (int)__builtin_rintf(q * 512.0f);
  } else {
    const int e = __builtin_amdgcn_frexp_expf(q) - 1;     // q in [2^e, 2^(e+1))
    const float r = __builtin_rintf(__builtin_ldexpf(q, 3 - e));
    c = min((e + 6) * 8 + (int)r, 0x7E);
  }
  int up = 0, down = 0;
  if (c < 0x7E) {  // beyond the midpoint to c + 1 (ties to the even code)
    const float M = 3.0f * (e4m3_value((uint32_t)c) + e4m3_value((uint32_t)c + 1u));
    const int r = cmp_scaled(amax, g, M);
    up = r > 0 || (r == 0 && ((c + 1) & 1) == 0);
  }
  if (c > 0) {     // below the midpoint to c - 1
    const float M = 3.0f * (e4m3_value((uint32_t)c - 1u) + e4m3_value((uint32_t)c));
    const int r = cmp_scaled(amax, g, M);
    down = r < 0 || (r == 0 && (c & 1) == 1);
  }
  return (uint32_t)(c + up - down);
}

// The seven decision boundaries between consecutive E2M1 magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} for block scale s and global scale g, as
// floats c[i] such that  magnitude code = #{ i : xs * |x| > c[i] }.
// The real boundaries are b_i = t_i * s * g with t = .25 .75 1.25 1.75 2.5
// 3.5 5.  A tie goes to the even code: up at .75, 1.75, 3.5 (c = the float
// below RU(b), so |x| > c <=> |x| >= b) and down at the others (c = RD(b),
// so |x| > c <=> |x| > b).  With b = p + e split exactly (t * s has at most
// 7 significant bits): RD(b) = p if e >= 0 else the float below p, and the
// float below RU(b) = p if e > 0 else the float below p.  For g < 2^-80 the
// bounds are those of 2^64 g and xs = 2^64 lifts |x| the same way (exact).
struct E2M1Bounds {
  float c0, c1, c2, c3, c4, c5, c6;
  float xs;
};
__device__ __forceinline__ float bound_rd(float g, float T) {
  const float p = g * T, e = __builtin_fmaf(g, T, -p);
  return e >= 0.0f ? p : __int_as_float(__float_as_int(p) - 1);
}
__device__ __forceinline__ float bound_below_ru(float g, float T) {
  const float p = g * T, e = __builtin_fmaf(g, T, -p);
  return e > 0.0f ? p : __int_as_float(__float_as_int(p) - 1);
}
__device__ __forceinline__ E2M1Bounds e2m1_bounds(float s, float g) {
  E2M1Bounds b;
  b.xs = 1.0f;
  if (g < kTinyG) {
    g *= kLift;
    b.xs = kLift;
  }
  b.c0 = bound_rd(g, 0.25f * s);
  b.c1 = bound_below_ru(g, 0.75f * s);
  b.c2 = bound_rd(g, 1.25f * s);
  b.c3 = bound_below_ru(g, 1.75f * s);
  b.c4 = bound_rd(g, 2.5f * s);
  b.c5 = bound_below_ru(g, 3.5f * s);
  b.c6 = bound_rd(g, 5.0f * s);
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
  const uint32_t mag = zero_scale ? 0u : e2m1_mag_code(fabsf(x) * b.xs, b);
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

// Load of a value that is the same for the whole wavefront and not written
// by the running kernel, through the scalar data cache (read-only use).  Its
// wait uses the scalar counter, so it never drains outstanding vector loads.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)ptr;
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (1 ulp) in place of
// an IEEE division.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Token of pair f: routed pairs are f = t*topk + j, shared pairs f = T*topk + t.
__device__ __forceinline__ int pair_token(int f, int T, int topk) {
  const int tk = T * topk;
  return f < tk ? f / topk : f - tk;
}

}  // namespace nvfp4
