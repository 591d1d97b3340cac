// OCP MXFP4 path for gfx950: E2M1 elements with one E8M0 (power of two)
// scale per 32 elements.  Here the block granularity and scale type match the
// scaled FP4 matrix instruction (16x16x128, one E8M0 scale per 32 k per
// operand row), so the codes feed the matrix unit as stored: no decoding.
//
// Quantisation (the format's usual definition; the pages only name OCP MX as
// the emulation backend's other format, vLLM PR #35737): scale
// 2^(floor(log2 amax) - 2), elements rounded to the nearest E2M1 value of
// v / scale (exact), ties to the even code, saturating at 6.
#include <algorithm>

#include "common.h"
#include "launch.h"
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
//
// FRAG = false: canonical output (codes [rows][K/2], bytes [rows][K/32]).
// FRAG = true: the operand layout the GEMM kernels read (K % 128 == 0, rows
// padded to rows_pad, a multiple of 64, with zeros): codes
// [rows_pad/16][K/128][64 lanes][16 B] (lane 16 g + m: row 16 t + m of row
// tile t, k in [32 g, 32 g + 32) of the chunk) and scale words
// [rows_pad/64][K/128][64 lanes][4 B] (byte t % 4: row tile t of the group),
// so that one instruction operand is 1 KiB contiguous and the scales of 4
// row tiles are one 256-byte run.
template <typename T, bool FRAG>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const T* __restrict__ x, int64_t rows, int64_t K,
                                                          int64_t ldx, int64_t rows_pad, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ ex) {
  const int64_t hb_per_row = K >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (FRAG ? rows_pad : rows) * hb_per_row) return;   // whole quads leave together
  const int64_t row = i / hb_per_row;
  const int64_t c8 = (i - row * hb_per_row) << 3;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (!FRAG || row < rows) load8(x, row * ldx + c8, v);   // (padding rows: zeros)
  int code;
  const uint32_t word = mx_encode8(v, code);
  if constexpr (FRAG) {
    const int64_t KC = K >> 7, t = row >> 4, kc = c8 >> 7;
    const int64_t lane = ((c8 & 127) >> 5) * 16 + (row & 15);
    *reinterpret_cast<uint32_t*>(q + ((t * KC + kc) * 64 + lane) * 16 + ((c8 & 31) >> 1)) = word;
    if ((c8 & 31) == 0) ex[((t >> 2) * KC + kc) * 256 + lane * 4 + (t & 3)] = (uint8_t)code;
  } else {
    *reinterpret_cast<uint32_t*>(q + row * (K >> 1) + (c8 >> 1)) = word;
    if ((c8 & 31) == 0) ex[row * (K >> 5) + (c8 >> 5)] = (uint8_t)code;
  }
}

// Weight streaming layout: codes [N/16][K/128][64 lanes][16 B] as for NVFP4
// (lane l = 16g + n: column n of the tile, k in [32g, 32g + 32) of the
// chunk: exactly the operand of the lane in the 16x16x128 instruction), then
// scale words [N/64][K/128][64 lanes][4 B]: byte t of lane l's word is the
// E8M0 byte of that lane in column tile 4q + t of group q.
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
  prep[N * (K / 2) + ((nt >> 2) * KC + kc) * 256 + lane * 4 + (nt & 3)] = ex[n * (K / 32) + kc * 4 + g];
}

// Byte offset, within the scale words, of lane l's E8M0 byte of column tile nt, chunk kc.
__device__ __forceinline__ int64_t mx_scale_at(int64_t nt, int64_t kc, int64_t KC, int lane) {
  return ((nt >> 2) * KC + kc) * 256 + lane * 4 + (nt & 3);
}

// y = x_hat W_hat^T for many rows.  Workgroup: 128 WM rows x 256 columns,
// 4 WM wavefronts of 128 x 64 (8 x 4 instruction tiles; WM = 2 puts two
// wavefronts on each SIMD and halves the weight bytes per product).  Both
// operands travel from global memory straight into a ring of D LDS stages
// (one chunk of 128 k each, no registers in between), D - 1 chunks in
// flight.  Each 1 KiB direct load fills one instruction operand in lane
// order (lane l's 16 bytes at 16 l) from 1 KiB of contiguous source (the
// activation operand layout and the weight streaming layout), so every load
// uses whole cache lines and every fragment read is conflict-free.
//
// Stage layout (bytes): activation tiles 8 WM x 1 KiB (tile i, lane l =
// 16 g + m: row 16 i + m, codes k in [32 g, 32 g + 32)), activation scale
// words 4 x 256 (group q: row tiles 4 q .. 4 q + 3, lane l's word, byte
// i % 4), weight tiles 16 x 1 KiB (column tile j of the workgroup), weight
// scale words 4 x 256 (group q: column tiles 4 q .. 4 q + 3).
// Loads per wavefront per chunk: 2 activation tiles, 16 / (4 WM) weight
// tiles and one run of scale words (WM = 1: the activation groups are
// loaded twice, into slots that are not read).
//
// Tile order: workgroups are dealt to the 8 XCDs in turn (workgroup b runs on
// XCD b % 8), and each XCD has its own L2.  Workgroup b takes tile
// (b % 8) * ceil(tiles / 8) + b / 8 of a list that walks groups of GM row
// tiles column tile by column tile, so the workgroups resident on one XCD
// share a few weight column tiles and a few activation row tiles.
#ifndef NVFP4_MX_DEPTH
#define NVFP4_MX_DEPTH 4
#endif
#ifndef NVFP4_MX_GM
#define NVFP4_MX_GM 8
#endif

template <int WM>
struct MxRing {
  static constexpr int A = 0, As = 8192 * WM, B = As + 1024 + 1024 * (WM == 1), Bs = B + 16384, Slot = Bs + 1024;
  static constexpr int Loads = 2 + 4 / WM + (WM == 1 ? 2 : 1);   // direct loads per wavefront per chunk
};

// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (the LDS and export counters left at their maxima).
constexpr int mx_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int WM, int D, bool F32>
__global__ __launch_bounds__(256 * WM) __attribute__((amdgpu_waves_per_eu(WM, WM))) void mx_gemm_kernel(
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_e, int64_t M, int64_t N, int64_t K,
    const uint8_t* __restrict__ w_prep, void* __restrict__ out) {
  using R = MxRing<WM>;
  static_assert(D >= 2 && (D - 2) * R::Loads <= 63, "ring depth");
  constexpr int ROWS = 128 * WM, MT = 8, NTW = 4, NBW = 4 / WM;
  __shared__ __attribute__((aligned(16))) uint8_t ring[D * R::Slot];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int64_t TM = (M + ROWS - 1) / ROWS, TN = (N + 255) / 256, tiles = TM * TN;
  const int64_t per_xcd = (tiles + 7) / 8;
  const int64_t L = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L >= tiles) return;
  const int64_t grp = L / (NVFP4_MX_GM * TN);
  const int64_t gh = min((int64_t)NVFP4_MX_GM, TM - grp * NVFP4_MX_GM);
  const int64_t Lg = L - grp * NVFP4_MX_GM * TN;
  const int64_t tm = grp * NVFP4_MX_GM + Lg % gh, tn = Lg / gh;
  const int64_t m0 = tm * ROWS;
  const int64_t n_wave0 = tn * 256 + wn * 64;
  const bool wave_on = n_wave0 < N;
  const int KC = (int)(K / 128);

  // Per-lane 32-bit source offsets of this wavefront's loads (chunk 0);
  // chunk kc adds kc * 1024 (tiles) or kc * 256 (scale words) bytes.  The
  // activations are in the operand layout with rows padded to whole
  // workgroup tiles (zeros past M); column tiles past N repeat the last
  // group of 4 (loaded, never stored).
  uint32_t va[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) va[t] = (uint32_t)((((tm * 8 * WM + 2 * wv + t) * KC) * 64 + lane) * 16);
  uint32_t vb[NBW];
#pragma unroll
  for (int t = 0; t < NBW; ++t) {
    const int jt = wv * NBW + t;                                 // column tile of the workgroup
    const int64_t nt = min(tn * 16 + jt, N / 16 - 4 + (jt & 3));  // past N: the last group
    vb[t] = (uint32_t)(((nt * KC) * 64 + lane) * 16);
  }
  // scale words: WM = 1: wavefront w loads activation group (w & 1) and
  // weight group w; WM = 2: wavefronts 0-3 the activation groups, 4-7 the
  // weight groups.
  const int64_t nq_last = N / 64 - 1;
  const int qa = WM == 1 ? (wv & 1) : wv;
  const int qb = WM == 1 ? wv : wv - 4;
  const uint32_t vsa = (uint32_t)((((tm * 2 * WM + qa) * KC) * 64 + lane) * 4);
  const uint32_t vsb = (uint32_t)(((min(tn * 4 + qb, nq_last) * KC) * 64 + lane) * 4);
  const uint8_t* w_sc = w_prep + N * (K / 2);
  const uint32_t ring0 = (uint32_t)(uintptr_t)ring;

  // Issue chunk kc (clamped to the last) into ring slot `slot`.  Assembly:
  // the compiler would otherwise treat each direct load as a pending LDS
  // write that any later LDS read may alias and wait for all of them before
  // every fragment read, which would drain the ring.  Completion is awaited
  // explicitly (vmcnt) before the barrier that publishes a slot.
  auto issue = [&](int kc, int slot) {
    kc = min(kc, KC - 1);
    const uint32_t base = ring0 + (uint32_t)slot * R::Slot;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(va[t] + (uint32_t)kc * 1024u), "s"(a_q),
                   "{m0}"(base + R::A + (2 * wv + t) * 1024) : "memory");
#pragma unroll
    for (int t = 0; t < NBW; ++t)
      asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(vb[t] + (uint32_t)kc * 1024u), "s"(w_prep),
                   "{m0}"(base + R::B + (wv * NBW + t) * 1024) : "memory");
    if (WM == 1 || wv < 4)
      asm volatile("global_load_lds_dword %0, %1" : : "v"(vsa + (uint32_t)kc * 256u), "s"(a_e),
                   "{m0}"(base + R::As + wv * 256) : "memory");
    if (WM == 1 || wv >= 4)
      asm volatile("global_load_lds_dword %0, %1" : : "v"(vsb + (uint32_t)kc * 256u), "s"(w_sc),
                   "{m0}"(base + R::Bs + qb * 256) : "memory");
  };

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fg = lane >> 4;
  auto compute = [&](int slot) {
    const uint8_t* st = ring + slot * R::Slot;
    u32x4 b[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) b[j] = *reinterpret_cast<const u32x4*>(st + R::B + (wn * 4 + j) * 1024 + lane * 16);
    const uint32_t bsw = *reinterpret_cast<const uint32_t*>(st + R::Bs + wn * 256 + lane * 4);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int ti = wm * 8 + i;
      const u32x4 a = *reinterpret_cast<const u32x4*>(st + R::A + ti * 1024 + lane * 16);
      const uint32_t aw = *reinterpret_cast<const uint32_t*>(st + R::As + (ti >> 2) * 256 + lane * 4);
      const int as = (int)((aw >> (8 * (ti & 3))) & 0xFFu);
      const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const v8i bv = {(int)b[j][0], (int)b[j][1], (int)b[j][2], (int)b[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, as, 0,
                                                                    (int)((bsw >> (8 * j)) & 0xFFu));
      }
    }
  };

  // Ring: chunk c lives in slot c % D.  At the top of iteration c the
  // chunks c .. c + D - 2 are in flight (Loads each, in issue order); once
  // at most (D - 2) Loads remain, chunk c has landed.  The barrier then
  // publishes it and also guarantees that every wavefront has finished
  // reading slot (c - 1) % D, which is refilled with chunk c + D - 1.
#pragma unroll
  for (int c = 0; c < D - 1; ++c) issue(c, c);
  // (unrolled by D so that every slot index is a constant; compute runs also
  // on wavefronts past N: a branch around it costs accumulator copies)
  for (int c0 = 0; c0 < KC; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (c0 + d < KC) {
        __builtin_amdgcn_s_waitcnt(mx_vmcnt((D - 2) * R::Loads));
        __syncthreads();
        issue(c0 + d + D - 1, (d + D - 1) % D);
        compute(d);
      }
    }
  }
  // Drain the direct loads still in flight (chunks past the end) before the
  // workgroup's LDS can be handed to another workgroup.
  __builtin_amdgcn_s_waitcnt(mx_vmcnt(0));
  if (!wave_on) return;
  const int64_t mw0 = m0 + wm * 128;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = mw0 + i * 16 + fg * 4 + r;
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
  // (activations in the operand layout, rows padded with zeros to 64: row
  // tile i of chunk kc at ((i KC + kc) 64 + lane) 16, its scale byte i of
  // word (kc 64 + lane))
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
        bs[u][j] = w_sc[mx_scale_at(nt0 + j, kc, KC, lane)];
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        aq[u][i] = *reinterpret_cast<const u32x4*>(a_q + ((i * KC + kc) * 64 + lane) * 16);
        as[u][i] = a_e[(kc * 64 + lane) * 4 + i];
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

template <int WM>
hipError_t launch_mx_gemm_ring(const uint8_t* a_q, const uint8_t* a_e, int64_t M, int64_t N, int64_t K,
                               const uint8_t* w_prep, void* out, int out_dtype, hipStream_t s) {
  const int64_t tiles = ((M + 128 * WM - 1) / (128 * WM)) * ((N + 255) / 256);
  const unsigned grid = (unsigned)(8 * ((tiles + 7) / 8));
  if (out_dtype) mx_gemm_kernel<WM, NVFP4_MX_DEPTH, true><<<grid, 256 * WM, 0, s>>>(a_q, a_e, M, N, K, w_prep, out);
  else mx_gemm_kernel<WM, NVFP4_MX_DEPTH, false><<<grid, 256 * WM, 0, s>>>(a_q, a_e, M, N, K, w_prep, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Mixture-of-experts layer in OCP MXFP4 (the emulation backend's other block
// format, vLLM PR #35737, "Purpose"): grouped GEMMs on the scaled FP4 matrix
// instruction, tiles from the alignment plan of moe_align.
//
// Expert weights: one dense prepared matrix per expert slot (codes
// [N/16][K/128][64 lanes][16 B], then scale words [N/64][K/128][64 lanes]
// [4 B]), experts one after the other.  For the gate/up weights the column
// tiles alternate gate and up: tile 2 q holds gate rows [16 q, 16 q + 16),
// tile 2 q + 1 the matching up rows, so that a wavefront's 64 columns are the
// gate and up halves of 32 columns of h -- one MX block of the intermediate.
__global__ __launch_bounds__(256) void mx_expert_prep_kernel(int64_t N, int64_t K, int interleave_I,
                                                             const uint8_t* __restrict__ q,
                                                             const uint8_t* __restrict__ ex,
                                                             uint8_t* __restrict__ prep) {
  const int64_t KC = K / 128, NT = N / 16, e = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= NT * KC * 64) return;
  const int64_t lane = i & 63, rest = i >> 6;
  const int64_t kc = rest % KC, nt = rest / KC;
  const int64_t tile_row = interleave_I ? ((nt & 1) ? interleave_I + 16 * (nt >> 1) : 16 * (nt >> 1)) : nt * 16;
  const int64_t n = tile_row + (lane & 15), g = lane >> 4;
  const uint8_t* qe = q + e * N * (K / 2);
  const uint8_t* xe = ex + e * N * (K / 32);
  uint8_t* pe = prep + e * (N * (K / 2) + N * (K / 32));
  *reinterpret_cast<u32x4*>(pe + i * 16) = *reinterpret_cast<const u32x4*>(qe + n * (K / 2) + kc * 64 + 16 * g);
  pe[N * (K / 2) + ((nt >> 2) * KC + kc) * 256 + lane * 4 + (nt & 3)] = xe[n * (K / 32) + kc * 4 + g];
}

enum MxEpi { kMxSwiglu = 0, kMxStoreF32 = 1 };

struct MxMoeParams {
  int T, topk, N, K, I, list_idx, n_blocks;
  const int32_t* plan;
  const int32_t* sorted_pair;   // GEMM1: row -> pair (activation row = its token); GEMM2: null
  const uint8_t* a_q;           // canonical codes [rows][K/2]
  const uint8_t* a_e;           // canonical exponent bytes [rows][K/32]
  const uint8_t* w_prep;        // experts' prepared weights
  int64_t w_expert_bytes;
  uint8_t* out_q;               // GEMM1: a2 codes [P][I/2]
  uint8_t* out_e;               // GEMM1: a2 exponent bytes [P][I/32]
  float* out_f32;               // GEMM2: d [P][N]
};

// Stage of the LDS ring: MT activation tiles (1 KiB: lane 16 g + m holds row
// m's codes k in [32 g, 32 g + 32) of the chunk), MT words runs (256 B:
// lane l's 4 exponent bytes of row l % 16 for the chunk's 4 blocks), 16
// weight tiles (1 KiB each, the streaming layout) and 4 weight scale runs.
template <int MT>
struct MxMoeRing {
  static constexpr int A = 0, Ae = 1024 * MT, B = Ae + 256 * MT, Bs = B + 16384, Slot = Bs + 1024;
  static constexpr int D = MT == 4 ? 3 : 4;                       // stages (LDS: 2 workgroups per CU up to MT 4)
  // activation tiles issued by wavefront w: w, w + 4, ... (< MT)
  static constexpr int a_per_wave(int w) { return MT >= 4 ? MT / 4 : (w < MT ? 1 : 0); }
  static constexpr int loads(int w) { return 2 * a_per_wave(w) + 4 + 1; }
};

// Epilogue of one wavefront (64 columns: column tiles nt_wave .. nt_wave + 3)
// for the row groups i < MTA of its accumulators.
//   kMxStoreF32: FP32 rows of the down projection into the workspace.
//   kMxSwiglu: the tiles are (gate, up, gate, up): h columns 32 w + fr and
//   32 w + 16 + fr of MX block w; a row's 32 values sit on the 16 lanes of
//   one DPP row, so the block amax is a row maximum, the exponent byte is
//   frexp(amax) - 3 + 127 (clamped; 0 for an all-zero block) and each code is
//   7 threshold comparisons of the exactly scaled value.
template <int MTA, int MTACC, int EPI>
__device__ __forceinline__ void mx_epilogue(const MxMoeParams& p, const f32x4 (&acc)[MTACC][4], int row0,
                                            int nrows, int nt_wave, int lane) {
  const int N = p.N;
  const int fr = lane & 15, fg = lane >> 4;
  if constexpr (EPI == kMxStoreF32) {
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + fg * 4 + r;
          if (row < nrows)
            p.out_f32[(int64_t)(row0 + row) * N + (nt_wave + j) * 16 + fr] = acc[i][j][r];
        }
  } else {
    const int w = nt_wave >> 2;
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float h0 = silu_fast(acc[i][0][r]) * acc[i][1][r];
        const float h1 = silu_fast(acc[i][2][r]) * acc[i][3][r];
        const float am = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
        const int code = am > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(am) - 1 - 2 + 127, 0), 254) : 0;
        const int sh = 127 - code;
        uint32_t c[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float hv = u == 0 ? h0 : h1;
          const float a = fabsf(__builtin_ldexpf(hv, sh));   // exact: a power-of-two scaling
          const uint32_t mag = (uint32_t)(a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                               (a >= 3.5f) + (a > 5.0f);
          c[u] = (((uint32_t)__float_as_int(hv) >> 28) & 8u) | mag;
        }
        const uint32_t o0 = (uint32_t)dpp_xor1_i((int)c[0]), o1 = (uint32_t)dpp_xor1_i((int)c[1]);
        const int row = i * 16 + fg * 4 + r;
        if (row < nrows) {
          const int64_t pr = row0 + row;
          if ((fr & 1) == 0) {
            p.out_q[pr * (p.I >> 1) + (32 * w + fr) / 2] = (uint8_t)(c[0] | (o0 << 4));
            p.out_q[pr * (p.I >> 1) + (32 * w + 16 + fr) / 2] = (uint8_t)(c[1] | (o1 << 4));
          }
          if (fr == 0) p.out_e[pr * (p.I >> 5) + w] = (uint8_t)code;
        }
      }
  }
}

// FP32 row store of the down projection through a wave-private LDS tile
// (the tall-tile kernel): each 16-row group is turned around in two halves
// of 8 rows (8 x 68 floats), so that a lane stores 4 consecutive columns
// and the wavefront writes 256 contiguous bytes per row, instead of the
// 64-byte row pieces of the accumulator layout.
template <int MTA>
__device__ __forceinline__ void mx_epilogue_f32_lds(const MxMoeParams& p, const f32x4 (&acc)[MTA][4], int row0,
                                                    int nrows, int nt_wave, int lane, float* __restrict__ tile) {
  constexpr int LD = 68;   // row stride in floats: the two row quads of a write fall in distinct banks
  const int fr = lane & 15, fg = lane >> 4;
  const int rr = lane >> 4, c4 = (lane & 15) * 4;
  const int64_t N = p.N;
#pragma unroll
  for (int i = 0; i < MTA; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((fg >> 1) == h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) tile[((fg & 1) * 4 + r) * LD + j * 16 + fr] = acc[i][j][r];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        const int rl = ps * 4 + rr;
        const int row = i * 16 + 8 * h + rl;
        const f32x4 v = *reinterpret_cast<const f32x4*>(tile + rl * LD + c4);
        if (row < nrows) *reinterpret_cast<f32x4*>(p.out_f32 + (int64_t)(row0 + row) * N + nt_wave * 16 + c4) = v;
      }
      // (the next half rewrites the tile only after every lane has read it)
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// SwiGLU epilogue through a wave-private LDS tile (the tall-tile kernel,
// whose activation buffers are free once its last chunk is done): h of one
// 16-row group (16 rows x 32 columns, one MX block per row) is written in the
// accumulator layout and read back so that lane 4 row + q owns columns
// [8 q, 8 q + 8) of its row.  The block amax is then a local maximum and two
// quad exchanges, and each lane stores its 8 codes as one 32-bit word (16
// contiguous bytes per row) instead of single bytes.  Same decisions as
// mx_epilogue: the maximum is exact and the per-value rule is the same.
template <int MTA, int MTACC>
__device__ __forceinline__ void mx_epilogue_swiglu_lds(const MxMoeParams& p, const f32x4 (&acc)[MTACC][4],
                                                       int row0, int nrows, int nt_wave, int lane,
                                                       float* __restrict__ tile) {
  constexpr int LD = 36;   // row stride in floats: the 4 row groups of a write fall in distinct banks
  const int fr = lane & 15, fg = lane >> 4;
  const int w = nt_wave >> 2;
  const int rr = lane >> 2, q = lane & 3;
#pragma unroll
  for (int i = 0; i < MTA; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tile[(fg * 4 + r) * LD + fr] = silu_fast(acc[i][0][r]) * acc[i][1][r];
      tile[(fg * 4 + r) * LD + 16 + fr] = silu_fast(acc[i][2][r]) * acc[i][3][r];
    }
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(tile + rr * LD + 8 * q);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(tile + rr * LD + 8 * q + 4);
    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
    am = fmaxf(am, dpp_xor1(am));
    am = fmaxf(am, dpp_xor2(am));
    const int code = am > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(am) - 1 - 2 + 127, 0), 254) : 0;
    const int sh = 127 - code;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fabsf(__builtin_ldexpf(v[j], sh));   // exact: a power-of-two scaling
      const uint32_t mag = (uint32_t)(a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                           (a >= 3.5f) + (a > 5.0f);
      word |= ((((uint32_t)__float_as_int(v[j]) >> 28) & 8u) | mag) << (4 * j);
    }
    const int row = i * 16 + rr;
    if (row < nrows) {
      const int64_t pr = row0 + row;
      *reinterpret_cast<uint32_t*>(p.out_q + pr * (p.I >> 1) + 16 * w + 4 * q) = word;
      if (q == 0) p.out_e[pr * (p.I >> 5) + w] = (uint8_t)code;
    }
  }
}

template <int MT, int EPI>
__global__ __launch_bounds__(256) void grouped_mx_kernel(MxMoeParams p) {
  using R = MxMoeRing<MT>;
  constexpr int D = R::D, NTW = 4;
  __shared__ __attribute__((aligned(16))) uint8_t ring[D * R::Slot];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Tile of the plan list (consecutive work items on one XCD).
  const int ntiles = ld_uniform(p.plan + p.list_idx);
  const int G = ntiles * p.n_blocks;
  if ((int)blockIdx.x >= G) return;
  int v;
  {
    const int q = G >> 3, r = G & 7, x = blockIdx.x & 7, idx = blockIdx.x >> 3;
    v = x * q + min(x, r) + idx;
  }
  const int tile = v / p.n_blocks, nb = v - tile * p.n_blocks;
  const int* ent = p.plan + ld_uniform(p.plan + kPlanLists + p.list_idx) + 2 * tile;
  const int e = ld_uniform(ent) & 2047;
  const uint32_t rr = (uint32_t)ld_uniform(ent + 1);
  const int row0 = (int)(rr & 0xFFFFFFu), nrows = (int)(rr >> 24);
  const int K = p.K, KC = K / 128, N = p.N, NT = N / 16;
  const int nt_wave = nb * 16 + wv * 4;                 // first column tile of this wavefront
  const bool wave_on = nt_wave * 16 < N;
  const int m = lane & 15, g = lane >> 4;

  // Per-lane source offsets (chunk 0).  Rows past the tile end repeat its
  // last valid row (loaded, never stored); column tiles past N repeat the
  // last group of four.
  constexpr int AW = MT >= 4 ? MT / 4 : 1;
  uint32_t va[AW], vae[AW];
#pragma unroll
  for (int u = 0; u < AW; ++u) {
    const int i = MT >= 4 ? wv + 4 * u : wv;            // activation tile this lane loads
    int r = row0 + min(16 * min(i, MT - 1) + m, nrows - 1);
    if (p.sorted_pair) r = pair_token(p.sorted_pair[r], p.T, p.topk);
    va[u] = (uint32_t)r * (uint32_t)(K / 2) + (uint32_t)(16 * g);
    vae[u] = (uint32_t)r * (uint32_t)(K / 32);
  }
  const uint8_t* wq = p.w_prep + (int64_t)e * p.w_expert_bytes;
  const uint8_t* ws = wq + (int64_t)N * (K / 2);
  uint32_t vb[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int nt = min(nt_wave + t, NT - 4 + t);
    vb[t] = (uint32_t)((nt * KC) * 64 + lane) * 16u;
  }
  const uint32_t vbs = (uint32_t)((min(nt_wave, NT - 4) / 4 * KC) * 64 + lane) * 4u;
  const uint32_t ring0 = (uint32_t)(uintptr_t)ring;

  // Issue chunk kc (clamped to the last) into ring slot `slot`: direct loads
  // (assembly, see mx_gemm_kernel), awaited with explicit vmcnt waits.
  auto issue = [&](int kc, int slot) {
    kc = min(kc, KC - 1);
    const uint32_t base = ring0 + (uint32_t)slot * R::Slot;
    if (R::a_per_wave(wv) > 0) {
#pragma unroll
      for (int u = 0; u < AW; ++u) {
        const int i = MT >= 4 ? wv + 4 * u : wv;
        asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(va[u] + (uint32_t)kc * 64u), "s"(p.a_q),
                     "{m0}"(base + R::A + i * 1024) : "memory");
        asm volatile("global_load_lds_dword %0, %1" : : "v"(vae[u] + (uint32_t)kc * 4u), "s"(p.a_e),
                     "{m0}"(base + R::Ae + i * 256) : "memory");
      }
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(vb[t] + (uint32_t)kc * 1024u), "s"(wq),
                   "{m0}"(base + R::B + (wv * NTW + t) * 1024) : "memory");
    asm volatile("global_load_lds_dword %0, %1" : : "v"(vbs + (uint32_t)kc * 256u), "s"(ws),
                 "{m0}"(base + R::Bs + wv * 256) : "memory");
  };

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot) {
    const uint8_t* st = ring + slot * R::Slot;
    u32x4 b[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) b[j] = *reinterpret_cast<const u32x4*>(st + R::B + (wv * NTW + j) * 1024 + lane * 16);
    const uint32_t bsw = *reinterpret_cast<const uint32_t*>(st + R::Bs + wv * 256 + lane * 4);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(st + R::A + i * 1024 + lane * 16);
      // lane l holds the 4 exponent bytes of row l % 16; its operand's block is g
      const uint32_t aw = *reinterpret_cast<const uint32_t*>(st + R::Ae + i * 256 + lane * 4);
      const int as = (int)((aw >> (8 * g)) & 0xFFu);
      const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const v8i bv = {(int)b[j][0], (int)b[j][1], (int)b[j][2], (int)b[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, as, 0,
                                                                    (int)((bsw >> (8 * j)) & 0xFFu));
      }
    }
  };
  auto wait_ring = [&]() {
    // at most (D - 2) chunks' loads of this wavefront still in flight
    if (R::a_per_wave(wv) > 0) __builtin_amdgcn_s_waitcnt(mx_vmcnt((D - 2) * R::loads(0)));
    else __builtin_amdgcn_s_waitcnt(mx_vmcnt((D - 2) * R::loads(3)));
  };
#pragma unroll
  for (int c = 0; c < D - 1; ++c) issue(c, c);
  for (int c0 = 0; c0 < KC; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (c0 + d < KC) {
        wait_ring();
        __syncthreads();
        issue(c0 + d + D - 1, (d + D - 1) % D);
        compute(d);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(mx_vmcnt(0));
  if (!wave_on) return;

  mx_epilogue<MT, MT, EPI>(p, acc, row0, nrows, nt_wave, lane);
}

// Tall tiles (the 64- and 128-row plan lists) run on a kernel built for two
// workgroups per CU, i.e. two wavefronts per SIMD: one wavefront per SIMD
// leaves every LDS read latency and every barrier exposed, and with 16 chunks
// per tile (K = 2048; 6 for the down projection) a workgroup's ring fill and
// drain are not hidden by another one.  Each wavefront owns 64 columns, so
// no wavefront shares another's weights: they stream from memory straight
// into registers (the streaming layout is the instruction operand, one
// 16-byte load per lane per column tile and chunk) through a ring of three
// chunks.  The activation tile is shared by the four wavefronts: in the
// straight-line bodies its rows are gathered two chunks per load (128-byte
// row pieces) into registers and written to four LDS chunk buffers, each at
// least one chunk ahead of use; the looped body gathers one chunk two
// chunks ahead into two buffers.  Exponent words are kept as
// [row][tile] so that one 16-byte read gives a lane the bytes of 4 tiles.
// Every load is an ordinary one, so the compiler's own waits are exact.
// The main loop is instantiated for 8, 4, 2 and 1 active 16-row groups: a
// ragged last tile stages and multiplies only the groups that hold rows.
constexpr int kMxTallRing = 3;   // weight chunks in registers
constexpr int kMxTallBufs = 4;   // activation chunk buffers in LDS

// KCT > 0: the chunk loop fully unrolled for K = 128 KCT (straight-line code,
// so the compiler's waits are exact; in a loop its analysis merges the
// header's incoming states and falls back to draining every load).  KCT = 0:
// any K, as a loop.
template <int MTA, int EPI, int KCT>
__device__ __forceinline__ void mx_tall_body(const MxMoeParams& p, uint8_t (*sa)[8 * 1024], uint32_t (*se)[16 * 8],
                                             int e, int row0, int nrows, int nb) {
  constexpr int NTW = 4, AW = MTA >= 4 ? MTA / 4 : 1, RB = kMxTallRing;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, KC = KCT > 0 ? KCT : K / 128, N = p.N, NT = N / 16;
  const int nt_wave = nb * 16 + wv * 4;
  const bool wave_on = nt_wave * 16 < N;
  const int m = lane & 15, g = lane >> 4;
  const bool a_on = MTA >= 4 || wv < MTA;         // this wavefront stages activation tiles

  // Activation tile i = wv + 4 u (u < AW): lane 16 g + m loads row m, bytes
  // [16 g, 16 g + 16) of the chunk's 64; rows past the tile end repeat its
  // last row (loaded, never stored).  Each lane also loads the exponent word
  // (4 blocks of the chunk) of row m of tile wv + 4 min(g, AW - 1).
  uint32_t va[AW];
  int tok[AW];
#pragma unroll
  for (int u = 0; u < AW; ++u) {
    const int i = MTA >= 4 ? wv + 4 * u : min(wv, MTA - 1);
    int r = row0 + min(16 * i + m, nrows - 1);
    if (p.sorted_pair) r = pair_token(p.sorted_pair[r], p.T, p.topk);
    tok[u] = r;
    va[u] = (uint32_t)r * (uint32_t)(K / 2) + (uint32_t)(16 * g);
  }
  const int ge = min(g, AW - 1);
  const uint32_t vae = (uint32_t)tok[ge] * (uint32_t)(K / 32);
  const int ie = MTA >= 4 ? wv + 4 * ge : min(wv, MTA - 1);   // tile of this lane's exponent word

  const uint8_t* wq = p.w_prep + (int64_t)e * p.w_expert_bytes;
  const uint8_t* ws = wq + (int64_t)N * (K / 2);
  uint32_t vb[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int nt = min(nt_wave + t, NT - 4 + t);
    vb[t] = (uint32_t)((nt * KC) * 64 + lane) * 16u;
  }
  const uint32_t vbs = (uint32_t)((min(nt_wave, NT - 4) / 4 * KC) * 64 + lane) * 4u;

  u32x4 rb[RB][NTW];
  uint32_t rbs[RB];
  u32x4 ra[AW];
  uint32_t rae;
  // Whole-cache-line gathers (straight-line bodies): two chunks per load, lane
  // l taking row (l >> 3) + 8 h of its tile, bytes [16 (l & 3), +16) of chunk
  // kc0 + ((l >> 2) & 1), i.e. 128 contiguous bytes per row.
  constexpr bool PAIR = KCT > 0;
  static_assert(KCT % 2 == 0, "pair gathers take whole chunk pairs");
  const int half = (lane >> 2) & 1;
  uint32_t vrow[AW][2];
#pragma unroll
  for (int u = 0; u < AW; ++u) {
    const int i = MTA >= 4 ? wv + 4 * u : min(wv, MTA - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int r = row0 + min(16 * i + (lane >> 3) + 8 * h, nrows - 1);
      if (p.sorted_pair) r = pair_token(p.sorted_pair[r], p.T, p.topk);
      vrow[u][h] = (uint32_t)r * (uint32_t)(K / 2) + (uint32_t)(16 * (lane & 3));
    }
  }
  u32x4 rp[AW][2];
  auto load_pair = [&](int kc0) __attribute__((always_inline)) {
    if (!a_on) return;
    const int c = min(kc0 + half, KC - 1);
#pragma unroll
    for (int u = 0; u < AW; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) rp[u][h] = *reinterpret_cast<const u32x4*>(p.a_q + (vrow[u][h] + (uint32_t)c * 64u));
  };
  auto store_pair = [&](int kc0) __attribute__((always_inline)) {
    if (!a_on) return;
    uint8_t* const base = half ? sa[(kc0 + 1) % kMxTallBufs] : sa[kc0 % kMxTallBufs];
#pragma unroll
    for (int u = 0; u < AW; ++u) {
      const int i = MTA >= 4 ? wv + 4 * u : wv;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // fragment slot of (row, g) in a chunk of parity q: 16 g + (row ^ (2 g + q)),
        // so that the 8 lanes of one row piece land in distinct banks
        const int g4 = lane & 3, row = (lane >> 3) + 8 * h;
        *reinterpret_cast<u32x4*>(base + i * 1024 + (16 * g4 + (row ^ (2 * g4 + half))) * 16) = rp[u][h];
      }
    }
  };
  auto load_e = [&](int kc) __attribute__((always_inline)) {
    if (!a_on) return;
    kc = min(kc, KC - 1);
    rae = *reinterpret_cast<const uint32_t*>(p.a_e + (vae + (uint32_t)kc * 4u));
  };
  auto store_e = [&](int buf) __attribute__((always_inline)) {
    if (!a_on) return;
    se[buf][m * 8 + ie] = rae;
  };
  // Loads past the last chunk repeat it (unconditional, so every wait is
  // the same in every iteration).
  auto load_b = [&](int kc, u32x4 (&b)[NTW], uint32_t& bs) __attribute__((always_inline)) {
    kc = min(kc, KC - 1);
#pragma unroll
    for (int t = 0; t < NTW; ++t) b[t] = *reinterpret_cast<const u32x4*>(wq + (vb[t] + (uint32_t)kc * 1024u));
    bs = *reinterpret_cast<const uint32_t*>(ws + (vbs + (uint32_t)kc * 256u));
  };
  auto load_a = [&](int kc, u32x4 (&a)[AW], uint32_t& ae) __attribute__((always_inline)) {
    if (!a_on) return;
    kc = min(kc, KC - 1);
#pragma unroll
    for (int u = 0; u < AW; ++u) a[u] = *reinterpret_cast<const u32x4*>(p.a_q + (va[u] + (uint32_t)kc * 64u));
    ae = *reinterpret_cast<const uint32_t*>(p.a_e + (vae + (uint32_t)kc * 4u));
  };
  auto store_a = [&](int buf, const u32x4 (&a)[AW], uint32_t ae) __attribute__((always_inline)) {
    if (!a_on) return;
#pragma unroll
    for (int u = 0; u < AW; ++u) {
      const int i = MTA >= 4 ? wv + 4 * u : wv;
      *reinterpret_cast<u32x4*>(sa[buf] + i * 1024 + lane * 16) = a[u];
    }
    // lanes g >= AW hold the word of lane (m, AW - 1) and store the same
    // value to the same place (no branch, so the waits stay exact)
    se[buf][m * 8 + ie] = ae;
  };

  f32x4 acc[MTA][NTW];
#pragma unroll
  for (int i = 0; i < MTA; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, const u32x4 (&b)[NTW], uint32_t bsw, int par) __attribute__((always_inline)) {
    // this lane's fragment slot (the pair gathers store swizzled by chunk parity)
    const int slot = PAIR ? 16 * g + (m ^ (2 * g + par)) : lane;
    // exponent bytes of row m for tiles 0..7, byte g of word i
    const u32x4 ew0 = *reinterpret_cast<const u32x4*>(&se[buf][m * 8]);
    u32x4 ew1 = ew0;
    if constexpr (MTA > 4) ew1 = *reinterpret_cast<const u32x4*>(&se[buf][m * 8 + 4]);
    // One fragment read ahead of the matrix instructions that use it (the
    // scheduler is fenced so that it does not hoist all MTA reads and their
    // registers to the top).
    u32x4 an = *reinterpret_cast<const u32x4*>(sa[buf] + slot * 16);
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
      const u32x4 a = an;
      if (i + 1 < MTA) an = *reinterpret_cast<const u32x4*>(sa[buf] + (i + 1) * 1024 + slot * 16);
      const uint32_t aw = i < 4 ? ew0[i & 3] : ew1[i & 3];
      const int as = (int)((aw >> (8 * g)) & 0xFFu);
      const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const v8i bv = {(int)b[j][0], (int)b[j][1], (int)b[j][2], (int)b[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, as, 0,
                                                                    (int)((bsw >> (8 * j)) & 0xFFu));
      }
      asm volatile("" ::: "memory");   // keeps the next read from being hoisted further
    }
  };

  // Prologue: activations of chunk 0 into buffer 0, chunk 1 into the
  // registers, weights of chunks 0..RB-1.
  if constexpr (PAIR) {
    load_pair(0);
    store_pair(0);
    load_e(0);
    store_e(0);
    load_e(1);
  } else {
    load_a(0, ra, rae);
    store_a(0, ra, rae);
    load_a(1, ra, rae);
  }
#pragma unroll
  for (int c = 0; c < RB; ++c) load_b(c, rb[c], rbs[c]);
  __syncthreads();

  // Iteration c: buffer c % 2 holds chunk c and rb[c % RB] its weights; ra
  // holds chunk c + 1.  Per iteration the loads go out activations first,
  // then weights, so that the wait before the activation store (loads
  // complete in order) does not also wait for the weights issued with it.
  auto step = [&](int c, int d) __attribute__((always_inline)) {
    compute(PAIR ? d % kMxTallBufs : d & 1, rb[d % RB], rbs[d % RB], d & 1);
    // The matrix instructions touch no memory: without this the compiler
    // sinks all of them past the barriers to the end of the unrolled body
    // and spills the fragments they read.  An empty statement that reads
    // and writes the accumulators keeps each chunk's instructions here.
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) asm volatile("" : "+v"(acc[i][j]));
    if constexpr (PAIR) {
      store_e((d + 1) % kMxTallBufs);
      if (d & 1) store_pair(c + 1);
      load_e(c + 2);
      if (!(d & 1)) load_pair(c + 2);
    } else {
      store_a((d + 1) & 1, ra, rae);
      load_a(c + 2, ra, rae);
    }
    load_b(c + RB, rb[d % RB], rbs[d % RB]);
    __syncthreads();
  };
  if constexpr (KCT > 0) {
#pragma unroll
    for (int c = 0; c < KCT; ++c) step(c, c);
  } else {
    constexpr int U = 6;   // lcm(2, RB)
    static_assert(U % RB == 0 && U % 2 == 0, "unroll covers both rings");
    for (int c0 = 0; c0 < KC; c0 += U) {
#pragma unroll
      for (int d = 0; d < U; ++d)
        if (c0 + d < KC) step(c0 + d, d);
    }
  }
  if (!wave_on) return;
  if constexpr (EPI == kMxSwiglu)
    mx_epilogue_swiglu_lds<MTA, MTA>(p, acc, row0, nrows, nt_wave, lane,
                                     reinterpret_cast<float*>(&sa[0][0]) + wv * 16 * 36);
  else
    mx_epilogue_f32_lds<MTA>(p, acc, row0, nrows, nt_wave, lane, reinterpret_cast<float*>(&sa[0][0]) + wv * 8 * 68);
}

// The contraction lengths of the expert shapes get straight-line bodies.
template <int MTA, int EPI>
__device__ __forceinline__ void mx_tall_groups(const MxMoeParams& p, uint8_t (*sa)[8 * 1024],
                                               uint32_t (*se)[16 * 8], int e, int row0, int nrows, int nb) {
  switch (p.K) {
    case 768: mx_tall_body<MTA, EPI, 6>(p, sa, se, e, row0, nrows, nb); break;
    case 1024: mx_tall_body<MTA, EPI, 8>(p, sa, se, e, row0, nrows, nb); break;
    case 2048: mx_tall_body<MTA, EPI, 16>(p, sa, se, e, row0, nrows, nb); break;
    case 4096: mx_tall_body<MTA, EPI, 32>(p, sa, se, e, row0, nrows, nb); break;
    default: mx_tall_body<MTA, EPI, 0>(p, sa, se, e, row0, nrows, nb); break;
  }
}

template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_mx_tall_kernel(MxMoeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[kMxTallBufs][8 * 1024];
  __shared__ __attribute__((aligned(16))) uint32_t se[kMxTallBufs][16 * 8];
  const int ntiles = ld_uniform(p.plan + p.list_idx);
  const int G = ntiles * p.n_blocks;
  if ((int)blockIdx.x >= G) return;
  int v;
  {
    const int q = G >> 3, r = G & 7, x = blockIdx.x & 7, idx = blockIdx.x >> 3;
    v = x * q + min(x, r) + idx;
  }
  const int tile = v / p.n_blocks, nb = v - tile * p.n_blocks;
  const int* ent = p.plan + ld_uniform(p.plan + kPlanLists + p.list_idx) + 2 * tile;
  const int e = ld_uniform(ent) & 2047;
  const uint32_t rr = (uint32_t)ld_uniform(ent + 1);
  const int row0 = (int)(rr & 0xFFFFFFu), nrows = (int)(rr >> 24);
  const int groups = (nrows + 15) >> 4;
  if (groups > 4) mx_tall_groups<8, EPI>(p, sa, se, e, row0, nrows, nb);
  else if (groups > 2) mx_tall_groups<4, EPI>(p, sa, se, e, row0, nrows, nb);
  else if (groups > 1) mx_tall_groups<2, EPI>(p, sa, se, e, row0, nrows, nb);
  else mx_tall_groups<1, EPI>(p, sa, se, e, row0, nrows, nb);
}

template <int MT, int EPI>
hipError_t launch_grouped_mx_t(MxMoeParams p, int64_t list_len, hipStream_t s) {
  const int64_t G = list_len * p.n_blocks;
  const unsigned grid = (unsigned)std::max<int64_t>(8, (G + 7) / 8 * 8);
  grouped_mx_kernel<MT, EPI><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_grouped_mx_tall(MxMoeParams p, int64_t list_len, hipStream_t s) {
  const int64_t G = list_len * p.n_blocks;
  const unsigned grid = (unsigned)std::max<int64_t>(8, (G + 7) / 8 * 8);
  grouped_mx_tall_kernel<EPI><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// part (kPart*): the short- or the tall-expert list of a split layer; a layer
// that is not split runs whole under kPartShort and not at all under kPartTall.
template <int EPI>
hipError_t launch_grouped_mx(MxMoeParams p, const AlignShape& al, hipStream_t s, int part) {
  p.n_blocks = (p.N + 255) / 256;
  if (split_experts(al)) {
    // short experts on 16-row tiles, the tall ones (a shared expert) on the
    // tall-tile kernel, which reads their weights once per 128 rows
    if (part != kPartTall) {
      p.list_idx = 4;
      const hipError_t e = launch_grouped_mx_t<1, EPI>(p, al.list_len[4], s);
      if (e != hipSuccess || part == kPartShort) return e;
    }
    p.list_idx = 5;
    return launch_grouped_mx_tall<EPI>(p, al.list_len[5], s);
  }
  if (part == kPartTall) return hipSuccess;
  const int li = pick_list(al.P, al.slots);
  p.list_idx = li;
  switch (li) {
    case 0: return launch_grouped_mx_t<1, EPI>(p, al.list_len[0], s);
    case 1: return launch_grouped_mx_t<2, EPI>(p, al.list_len[1], s);
    default: return launch_grouped_mx_tall<EPI>(p, al.list_len[li], s);
  }
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, uint8_t* q,
                              uint8_t* ex, hipStream_t s) {
  const int64_t lanes = rows * (K / 8);
  if (lanes == 0) return hipSuccess;
  const unsigned grid = (unsigned)((lanes + 255) / 256);
  if (dtype == 0)
    mx_quantize_kernel<uint16_t, false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), rows, K, ldx, rows, q, ex);
  else
    mx_quantize_kernel<float, false><<<grid, 256, 0, s>>>(static_cast<const float*>(x), rows, K, ldx, rows, q, ex);
  return hipGetLastError();
}

// Rows of the activation operand: whole tiles of the kernel that runs (64
// rows for the split-K kernels, 128 or 256 for the ring kernel).
int64_t mx_rows_pad(int64_t M) { return M <= 0 ? 0 : M <= 64 ? 64 : M <= 128 ? 128 : (M + 255) / 256 * 256; }

hipError_t launch_mx_quantize_operand(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* ex,
                                      hipStream_t s) {
  const int64_t lanes = mx_rows_pad(M) * (K / 8);
  mx_quantize_kernel<uint16_t, true><<<(unsigned)((lanes + 255) / 256), 256, 0, s>>>(x, M, K, K, mx_rows_pad(M), q, ex);
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
  // up to 128 rows: one 128-row tile (4 wavefronts); more: 256-row tiles
  if (M <= 128) return launch_mx_gemm_ring<1>(a_q, a_e, M, N, K, w_prep, out, out_dtype, s);
  return launch_mx_gemm_ring<2>(a_q, a_e, M, N, K, w_prep, out, out_dtype, s);
}

}  // namespace nvfp4

namespace nvfp4 {

size_t mx_expert_prep_bytes(int64_t slots, int64_t N, int64_t K) {
  return (size_t)slots * (size_t)(N * (K / 2) + N * (K / 32));
}

hipError_t launch_mx_expert_prep(int64_t slots, int64_t N, int64_t K, int interleave_I, const uint8_t* q,
                                 const uint8_t* ex, uint8_t* prep, hipStream_t s) {
  const int64_t pieces = (N / 16) * (K / 128) * 64;
  const dim3 grid((unsigned)((pieces + 255) / 256), (unsigned)slots);
  mx_expert_prep_kernel<<<grid, 256, 0, s>>>(N, K, interleave_I, q, ex, prep);
  return hipGetLastError();
}

hipError_t launch_mx_gemm1_swiglu(const MxGemmArgs& a, hipStream_t s) {
  const AlignShape al = align_shape(a.T, a.topk, a.E, a.shared);
  MxMoeParams p{};
  p.T = a.T;
  p.topk = a.topk;
  p.N = 2 * a.I;
  p.K = a.H;
  p.I = a.I;
  p.plan = a.plan;
  p.sorted_pair = a.sorted_pair;
  p.a_q = a.a_q;
  p.a_e = a.a_e;
  p.w_prep = a.w_prep;
  p.w_expert_bytes = (int64_t)p.N * (p.K / 2) + (int64_t)p.N * (p.K / 32);
  p.out_q = a.out_q;
  p.out_e = a.out_e;
  return launch_grouped_mx<kMxSwiglu>(p, al, s, a.part);
}

hipError_t launch_mx_gemm2_combine(const MxGemmArgs& a, hipStream_t s) {
  const AlignShape al = align_shape(a.T, a.topk, a.E, a.shared);
  MxMoeParams p{};
  p.T = a.T;
  p.topk = a.topk;
  p.N = a.H;
  p.K = a.I;
  p.I = a.I;
  p.plan = a.plan;
  p.sorted_pair = nullptr;                // a2 rows are in sorted order
  p.a_q = a.a_q;
  p.a_e = a.a_e;
  p.w_prep = a.w_prep;
  p.w_expert_bytes = (int64_t)p.N * (p.K / 2) + (int64_t)p.N * (p.K / 32);
  p.out_f32 = a.d_ws;
  const hipError_t e = a.part == kPartCombine ? hipSuccess : launch_grouped_mx<kMxStoreF32>(p, al, s, a.part);
  if (e != hipSuccess || (a.part != kPartAll && a.part != kPartCombine)) return e;
  return launch_combine(a.d_ws, a.inv_pos, a.topk_w, a.T, a.topk, a.shared, a.H, a.out, a.out_dtype, s);
}

}  // namespace nvfp4
