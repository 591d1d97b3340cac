// OCP MXFP4 path for gfx950: E2M1 elements with one E8M0 (power of two)
// scale per 32 elements.  Here the block granularity and scale type match the
// scaled FP4 matrix instruction (16x16x128, one E8M0 scale per 32 k per
// operand row), so the codes feed the matrix unit as stored: no decoding.
//
// Quantisation (the format's usual definition; the pages only name OCP MX as
// the emulation backend's other format, vLLM PR #35737): scale
// 2^(floor(log2 amax) - 2), elements rounded to the nearest E2M1 value of
// v / scale (exact), ties to the even code, saturating at 6.
#include "common.h"
#include "mx.h"
#include "quant.h"

namespace nvfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

// Split-K configurations by row tiles (MT = 1, 2, 4): column tiles per
// workgroup and chunks loaded per batch.
#ifndef NVFP4_MX_NTW1
#define NVFP4_MX_NTW1 2
#endif
#ifndef NVFP4_MX_UB1
#define NVFP4_MX_UB1 5
#endif
#ifndef NVFP4_MX_NTW2
#define NVFP4_MX_NTW2 4
#endif
#ifndef NVFP4_MX_UB2
#define NVFP4_MX_UB2 2
#endif
#ifndef NVFP4_MX_NTW4
#define NVFP4_MX_NTW4 4
#endif
#ifndef NVFP4_MX_UB4
#define NVFP4_MX_UB4 1
#endif

// One lane per 8 elements; the 4 lanes of a 32-element block form a DPP
// quad (K % 32 == 0 and the grid starts at a multiple of 4).
template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const T* __restrict__ x, int64_t rows, int64_t K,
                                                          int64_t ldx, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ ex) {
  const int64_t hb_per_row = K >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * hb_per_row) return;   // whole quads leave together
  const int64_t row = i / hb_per_row;
  const int64_t c8 = (i - row * hb_per_row) << 3;
  float v[8];
  load8(x, row * ldx + c8, v);
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  m = fmaxf(m, dpp_xor1(m));
  m = fmaxf(m, dpp_xor2(m));
  // floor(log2 m) = frexp exponent - 1 (m = f * 2^E, f in [0.5, 1)).
  const int code = m > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(m) - 1 - 2 + 127, 0), 254) : 0;
  const int sh = 127 - code;   // v / scale = v * 2^sh, exact
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
  *reinterpret_cast<uint32_t*>(q + row * (K >> 1) + (c8 >> 1)) = word;
  if ((c8 & 31) == 0) ex[row * (K >> 5) + (c8 >> 5)] = (uint8_t)code;
}

// Weight streaming layout: codes [N/16][K/128][64 lanes][16 B] as for NVFP4
// (lane l = 16g + n: column n of the tile, k in [32g, 32g + 32) of the
// chunk), then scale bytes [N/16][K/128][64 lanes] (that lane's E8M0 byte):
// exactly the operand and scale of the lane in the 16x16x128 instruction.
__global__ __launch_bounds__(256) void mx_prep_kernel(int64_t N, int64_t K, const uint8_t* __restrict__ q,
                                                      const uint8_t* __restrict__ ex,
                                                      uint8_t* __restrict__ prep) {
  const int64_t KC = K / 128, NT = N / 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= NT * KC * 64) return;
  const int64_t lane = i & 63, rest = i >> 6;
  const int64_t kc = rest % KC, nt = rest / KC;
  const int64_t n = nt * 16 + (lane & 15), g = lane >> 4;
  *reinterpret_cast<u32x4*>(prep + i * 16) = *reinterpret_cast<const u32x4*>(q + n * (K / 2) + kc * 64 + 16 * g);
  prep[N * (K / 2) + i] = ex[n * (K / 32) + kc * 4 + g];
}

// y = x_hat W_hat^T.  Workgroup: 4 wavefronts x 64 columns, 16 MT rows.  The
// activation chunk (16 MT rows x 128 k: 64 code bytes + 4 scale bytes per
// row) is staged in LDS, double-buffered (rows 80 bytes apart: the 16 rows of
// a fragment read hit distinct banks); weights stream into two register sets.
constexpr int kMxRowB = 80;
template <int MT, bool F32>
__global__ __launch_bounds__(256) void mx_gemm_kernel(const uint8_t* __restrict__ a_q,
                                                      const uint8_t* __restrict__ a_e, int64_t M, int64_t N,
                                                      int64_t K, const uint8_t* __restrict__ w_prep,
                                                      void* __restrict__ out) {
  constexpr int ROWS = 16 * MT, NTW = 4;
  __shared__ __attribute__((aligned(16))) uint8_t Aq[2][ROWS * kMxRowB];
  __shared__ uint32_t Ae[2][ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * ROWS;
  const int64_t n_wave0 = (int64_t)blockIdx.x * 256 + wv * 64;
  const bool wave_on = n_wave0 < N;
  const int64_t KC = K / 128;
  const uint8_t* w_sc = w_prep + N * (K / 2);

  // A staging: piece p = 16 bytes of a row (4 per row), scale words by the
  // first ROWS threads.  Rows past M repeat row M - 1 (never stored).
  constexpr int PIECES = ROWS * 4, PER = (PIECES + 255) / 256;
  u32x4 a_reg[PER];
  uint32_t e_reg = 0;
  auto load_a = [&](int64_t kc) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int p = tid + 256 * u;
      if (p < PIECES) {
        const int64_t r = min(m0 + (p >> 2), M - 1);
        a_reg[u] = *reinterpret_cast<const u32x4*>(a_q + r * (K / 2) + kc * 64 + (p & 3) * 16);
      }
    }
    if (tid < ROWS) {
      const int64_t r = min(m0 + tid, M - 1);
      e_reg = *reinterpret_cast<const uint32_t*>(a_e + r * (K / 32) + kc * 4);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int p = tid + 256 * u;
      if (p < PIECES) *reinterpret_cast<u32x4*>(&Aq[buf][(p >> 2) * kMxRowB + (p & 3) * 16]) = a_reg[u];
    }
    if (tid < ROWS) Ae[buf][tid] = e_reg;
  };
  u32x4 bq[2][NTW];
  uint32_t bs[2][NTW];
  auto load_b = [&](int64_t kc, int set) {
    if (!wave_on) return;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int64_t unit = ((n_wave0 / 16 + j) * KC + kc) * 64 + lane;
      bq[set][j] = *reinterpret_cast<const u32x4*>(w_prep + unit * 16);
      bs[set][j] = w_sc[unit];
    }
  };
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fg = lane >> 4;
  auto compute = [&](int buf, int set) {
    if (!wave_on) return;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(&Aq[buf][(i * 16 + fr) * kMxRowB + fg * 16]);
      const int as = (int)((Ae[buf][i * 16 + fr] >> (8 * fg)) & 0xFFu);
      const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const v8i bv = {(int)bq[set][j][0], (int)bq[set][j][1], (int)bq[set][j][2], (int)bq[set][j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, as, 0,
                                                                    (int)bs[set][j]);
      }
    }
  };

  load_a(0);
  load_b(0, 0);
  store_a(0);
  __syncthreads();
  for (int64_t kc = 0;; kc += 2) {
    const bool more1 = kc + 1 < KC;
    if (more1) {
      load_a(kc + 1);
      load_b(kc + 1, 1);
    }
    compute(0, 0);
    if (more1) store_a(1);
    __syncthreads();
    if (!more1) break;
    const bool more2 = kc + 2 < KC;
    if (more2) {
      load_a(kc + 2);
      load_b(kc + 2, 0);
    }
    compute(1, 1);
    if (more2) store_a(0);
    __syncthreads();
    if (!more2) break;
  }
  if (!wave_on) return;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + i * 16 + fg * 4 + r;
        if (row < M) {
          const int64_t o = row * N + n_wave0 + 16 * j + fr;
          if constexpr (F32) static_cast<float*>(out)[o] = acc[i][j][r];
          else static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
        }
      }
}

// Few rows (M <= 16 MT): the weight stream decides the time, so the grid is
// wide and each wavefront keeps many loads in flight.  A workgroup owns NTW
// column tiles (16 NTW columns); its 4 wavefronts split K into quarters, each
// loading UB chunks of weights and activations (straight from global memory:
// the activations are small and stay in L2) before multiplying them, then
// the quarters are summed through LDS.
template <int MT, int NTW, int UB, bool F32>
__global__ __launch_bounds__(256) void mx_gemm_splitk_kernel(const uint8_t* __restrict__ a_q,
                                                             const uint8_t* __restrict__ a_e, int64_t M,
                                                             int64_t N, int64_t K,
                                                             const uint8_t* __restrict__ w_prep,
                                                             void* __restrict__ out) {
  __shared__ f32x4 red[3][MT][NTW][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int64_t KC = K / 128;
  const int64_t c_lo = KC * wv / 4, c_hi = KC * (wv + 1) / 4;
  const int64_t nt0 = (int64_t)blockIdx.x * NTW;
  const uint8_t* w_sc = w_prep + N * (K / 2);
  const uint8_t* arow[MT];
  const uint8_t* erow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t r = min((int64_t)(i * 16 + fr), M - 1);
    arow[i] = a_q + r * (K / 2) + fg * 16;
    erow[i] = a_e + r * (K / 32) + fg;
  }
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t c0 = c_lo; c0 < c_hi; c0 += UB) {
    u32x4 bq[UB][NTW], aq[UB][MT];
    uint32_t bs[UB][NTW], as[UB][MT];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int64_t kc = min(c0 + u, c_hi - 1);   // a repeated chunk is loaded but not used
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int64_t unit = ((nt0 + j) * KC + kc) * 64 + lane;
        bq[u][j] = *reinterpret_cast<const u32x4*>(w_prep + unit * 16);
        bs[u][j] = w_sc[unit];
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        aq[u][i] = *reinterpret_cast<const u32x4*>(arow[i] + kc * 64);
        as[u][i] = erow[i][kc * 4];
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (c0 + u < c_hi) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const v8i av = {(int)aq[u][i][0], (int)aq[u][i][1], (int)aq[u][i][2], (int)aq[u][i][3], 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            const v8i bv = {(int)bq[u][j][0], (int)bq[u][j][1], (int)bq[u][j][2], (int)bq[u][j][3], 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                        (int)as[u][i], 0, (int)bs[u][j]);
          }
        }
      }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) red[wv - 1][i][j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wv > 0) return;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      f32x4 v = acc[i][j];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const f32x4 o = red[w][i][j][lane];
        v[0] += o[0];
        v[1] += o[1];
        v[2] += o[2];
        v[3] += o[3];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = i * 16 + fg * 4 + r;
        if (row < M) {
          const int64_t o = row * N + (nt0 + j) * 16 + fr;
          if constexpr (F32) static_cast<float*>(out)[o] = v[r];
          else static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16_bits(v[r]);
        }
      }
    }
}

template <int MT, int NTW, int UB>
hipError_t launch_mx_splitk(const uint8_t* a_q, const uint8_t* a_e, int64_t M, int64_t N, int64_t K,
                            const uint8_t* w_prep, void* out, int out_dtype, hipStream_t s) {
  const dim3 grid((unsigned)(N / (16 * NTW)));
  if (out_dtype) mx_gemm_splitk_kernel<MT, NTW, UB, true><<<grid, 256, 0, s>>>(a_q, a_e, M, N, K, w_prep, out);
  else mx_gemm_splitk_kernel<MT, NTW, UB, false><<<grid, 256, 0, s>>>(a_q, a_e, M, N, K, w_prep, out);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mx_gemm_mt(const uint8_t* a_q, const uint8_t* a_e, int64_t M, int64_t N, int64_t K,
                             const uint8_t* w_prep, void* out, int out_dtype, hipStream_t s) {
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)((M + 16 * MT - 1) / (16 * MT)));
  if (out_dtype) mx_gemm_kernel<MT, true><<<grid, 256, 0, s>>>(a_q, a_e, M, N, K, w_prep, out);
  else mx_gemm_kernel<MT, false><<<grid, 256, 0, s>>>(a_q, a_e, M, N, K, w_prep, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, uint8_t* q,
                              uint8_t* ex, hipStream_t s) {
  const int64_t lanes = rows * (K / 8);
  if (lanes == 0) return hipSuccess;
  const unsigned grid = (unsigned)((lanes + 255) / 256);
  if (dtype == 0)
    mx_quantize_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), rows, K, ldx, q, ex);
  else
    mx_quantize_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), rows, K, ldx, q, ex);
  return hipGetLastError();
}

size_t mx_prep_bytes(int64_t N, int64_t K) { return (size_t)(N * (K / 2) + N * (K / 32)); }

hipError_t launch_mx_prep(int64_t N, int64_t K, const uint8_t* q, const uint8_t* ex, uint8_t* prep,
                          hipStream_t s) {
  const int64_t pieces = (N / 16) * (K / 128) * 64;
  mx_prep_kernel<<<(unsigned)((pieces + 255) / 256), 256, 0, s>>>(N, K, q, ex, prep);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t* a_q, const uint8_t* a_e, int64_t M, int64_t N, int64_t K,
                          const uint8_t* w_prep, void* out, int out_dtype, hipStream_t s) {
  // N is a multiple of 128, so NTW <= 8 column tiles divide it.
  if (M <= 16) return launch_mx_splitk<1, NVFP4_MX_NTW1, NVFP4_MX_UB1>(a_q, a_e, M, N, K, w_prep, out, out_dtype, s);
  if (M <= 32) return launch_mx_splitk<2, NVFP4_MX_NTW2, NVFP4_MX_UB2>(a_q, a_e, M, N, K, w_prep, out, out_dtype, s);
  if (M <= 64) return launch_mx_splitk<4, NVFP4_MX_NTW4, NVFP4_MX_UB4>(a_q, a_e, M, N, K, w_prep, out, out_dtype, s);
  return launch_mx_gemm_mt<8>(a_q, a_e, M, N, K, w_prep, out, out_dtype, s);
}

}  // namespace nvfp4
