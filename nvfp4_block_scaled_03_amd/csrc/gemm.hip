// Grouped NVFP4 expert GEMMs with fused SwiGLU + requantisation (GEMM1) and
// the down projection + top-k weighted combine (GEMM2), for gfx950.
//
// Contraction strategy: NVFP4 operands are dequantised exactly (code * E4M3
// block scale has at most six significant bits and lies in [2^-10, 2688], so
// it is exact in f16) and multiplied on the 16x16x32 f16 (W4A4) or bf16
// (W4A16) matrix instructions with FP32 accumulation; the FP32 global scales
// enter as one per-expert alpha in the epilogue (the alpha-pointer-array
// epilogue with beta = 0 of vLLM PR #29242, review of
// nvfp4_blockwise_moe_kernel.cu).  The native FP4 matrix instructions of
// gfx950 take power-of-two scales per 32 elements, which cannot carry E4M3
// scales per 16 exactly.
//
// The FP4 conversion instructions of gfx950 issue at a quarter of the rate of
// plain VALU work, so decoding is the cost to minimise: every weight element
// is decoded once per wavefront that uses it, and the activations are either
// decoded once per workgroup (LDS kernel, codes in) or not at all (an exact
// f16 copy written by their producer: nvfp4_quantize for a1, the GEMM1
// epilogue for a2).  Activation kinds (template parameter AK):
//   kActCodes  NVFP4 codes + scales, decoded here
//   kActF16    the exact f16 dequantised copy of NVFP4 codes
//   kActBf16   bf16 activations (W4A16)
//
// Work decomposition: the alignment plan lists (expert, 16..128-row tile)
// pairs on the device.  Short tiles (the decode regime) run on a persistent
// streaming kernel; taller tiles on a kernel that stages the activation chunk
// in LDS once per workgroup.  Weights stream from HBM straight into registers
// in the layout written by prep.hip: one coalesced 16-byte load per lane per
// 16 columns x 128 k, which is exactly the lane's matrix-instruction operand.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

// Tile configuration (compile-time; the defaults are the measured best).
#ifndef NVFP4_LIST_MAX
#define NVFP4_LIST_MAX 2       // tallest tile list used (2: 64 rows, 3: 128 rows)
#endif
#ifndef NVFP4_BIG_WN
#define NVFP4_BIG_WN 32        // columns per wavefront, LDS-staged kernel
#endif
#ifndef NVFP4_BIG_NW
#define NVFP4_BIG_NW 4         // wavefronts per workgroup, LDS-staged kernel
#endif
#ifndef NVFP4_STREAM_NTW
#define NVFP4_STREAM_NTW 2     // 16-column tiles per work unit, streaming kernel (GEMM1)
#endif
#ifndef NVFP4_STREAM_NTW_DOWN
#define NVFP4_STREAM_NTW_DOWN 2  // the same for the down projection (GEMM2)
#endif
#ifndef NVFP4_WIDE_MIN_LIST
#define NVFP4_WIDE_MIN_LIST 2  // smallest tile list (by mean rows/expert) sent to the wide kernel
#endif

constexpr int kNW = 4;      // wavefronts per workgroup of the streaming kernel
constexpr int kBK = 128;    // contraction chunk
constexpr int kLDA = kBK + 8;  // LDS row stride in 16-bit elements (272 bytes)
// Word 3 of a raw buffer descriptor on gfx9 parts (32-bit data format, no
// swizzle, no index stride).
constexpr int kBufferFlags = 0x00020000;

enum Act { kActCodes = 0, kActF16 = 1, kActBf16 = 2 };
enum Epi { kEpiSwigluFp4 = 0, kEpiSwigluBf16 = 1, kEpiStoreF32 = 2, kEpiStoreBf16 = 3 };
constexpr bool swiglu_epi(int e) { return e == kEpiSwigluFp4 || e == kEpiSwigluBf16; }


struct KParams {
  int T, topk, I, N, K;
  int n_blocks;
  int list_idx;            // which plan list (tile height)
  int64_t a_rows;          // rows of the activation operand (T for GEMM1, P for GEMM2)
  const int32_t* sorted_pair;  // GEMM1: row -> pair; GEMM2: null (row is the A row)
  const int32_t* plan;
  const uint8_t* a_q;      // kActCodes
  const uint8_t* a_sf;
  const uint16_t* a_h;     // kActF16 / kActBf16: 16-bit activations [a_rows][K]
  const float* g_a;
  const uint8_t* w_q;      // prepped codes
  const uint8_t* w_sf;     // prepped scales
  const float* g_w;
  const float* g2;
  uint8_t* out_q;
  uint8_t* out_sf;
  uint16_t* out_h;         // GEMM1: bf16 intermediate (W4A16) or optional f16 copy (W4A4)
  float* out_f32;
};

// Bijection from the launch order to the work order such that each XCD (the
// hardware deals workgroups round-robin over 8 XCDs) receives a contiguous
// range of work items.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int q = G >> 3, r = G & 7, x = bid & 7, idx = bid >> 3;
  return x * q + min(x, r) + idx;
}


// Value of an E2M1 magnitude code 0..7: {0, .5, 1, 1.5, 2, 3, 4, 6}.
__device__ __forceinline__ float e2m1_mag_value(uint32_t m) {
  const float lo = (float)(m & 1u) * 0.5f;                        // codes 0, 1
  const float v = __int_as_float((int)(((m >> 1) + 126u) << 23)) * (1.0f + 0.5f * (float)(m & 1u));
  return m < 2 ? lo : v;                                          // 2^(e-1) * (1 + m/2)
}

// Epilogue of a wavefront's MT x NTW accumulator tiles (rows row0 + [0, 16 MT),
// columns n_wave0 + [0, 16 NTW) of the streaming column order).
template <int EPI, int MT, int NTW>
__device__ __forceinline__ void epilogue(const KParams& p, f32x4 (&acc)[MT][NTW], int e, int row0,
                                         int nrows, int n_wave0, int lane) {
  const float alpha = p.g_a ? ld_uniform(p.g_a) * ld_uniform(p.g_w + e) : ld_uniform(p.g_w + e);
  const int ln = lane & 15, lg = lane >> 4;
  if constexpr (EPI == kEpiStoreF32 || EPI == kEpiStoreBf16) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + lg * 4 + r;
          if (row < nrows) {
            const int64_t o = (int64_t)(row0 + row) * p.N + n_wave0 + 16 * j + ln;
            if constexpr (EPI == kEpiStoreF32)
              p.out_f32[o] = alpha * acc[i][j][r];
            else
              p.out_h[o] = (uint16_t)f32_to_bf16_bits(alpha * acc[i][j][r]);
          }
        }
  } else {
    const float g2 = (EPI == kEpiSwigluFp4) ? ld_uniform(p.g2) : 0.0f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < NTW / 2; ++q) {
        const int hb = (n_wave0 >> 5) + q;  // 16-column block of h
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gate = alpha * acc[i][2 * q][r];
          const float up = alpha * acc[i][2 * q + 1][r];
          h[r] = silu_fast(gate) * up;
        }
        if constexpr (EPI == kEpiSwigluFp4) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float am = row16_max(fabsf(h[r]));
            const uint32_t sc = e4m3_scale_code(am, g2);
            const float sv = e4m3_value(sc);
            const E2M1Bounds bd = e2m1_bounds(sv, g2);
            const uint32_t code = e2m1_code(h[r], bd, sc == 0);
            const uint32_t other = (uint32_t)dpp_xor1_i((int)code);
            const int row = i * 16 + lg * 4 + r;
            if (row < nrows) {
              const int64_t pr = row0 + row;
              if ((ln & 1) == 0)
                p.out_q[pr * (p.I >> 1) + hb * 8 + (ln >> 1)] = (uint8_t)(code | (other << 4));
              if (ln == 0) p.out_sf[pr * (p.I >> 4) + hb] = (uint8_t)sc;
              if (p.out_h) {
                // Exact: six significant bits at most, inside the f16 range.
                const float dv = e2m1_mag_value(code & 7u) * sv;
                const _Float16 hv = (_Float16)((code & 8u) ? -dv : dv);
                p.out_h[pr * p.I + hb * 16 + ln] = __builtin_bit_cast(uint16_t, hv);
              }
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = i * 16 + lg * 4 + r;
            if (row < nrows)
              p.out_h[(int64_t)(row0 + row) * p.I + hb * 16 + ln] = (uint16_t)f32_to_bf16_bits(h[r]);
          }
        }
      }
  }
}

// Row-major store epilogue (FP32 or bf16 output) of a wavefront's MT x NTW
// accumulator tiles through a wave-private LDS area sh of 16 x (16 NTW + 4)
// floats.  In the matrix-instruction layout a lane holds four rows of one
// column, so direct stores write 4 bytes per lane; here each 16-row m-tile
// is turned around in LDS and leaves as 16-byte (FP32) or 8-byte (bf16)
// stores of four consecutive columns, a wavefront writing whole rows.
template <int EPI, int MT, int NTW>
__device__ __forceinline__ void epilogue_rowmajor(const KParams& p, f32x4 (&acc)[MT][NTW], int e,
                                                  int row0, int nrows, int n_wave0, int lane,
                                                  float* sh) {
  static_assert(EPI == kEpiStoreF32 || EPI == kEpiStoreBf16, "plain stores only");
  constexpr int W = 16 * NTW;       // columns of the wavefront
  constexpr int SW = W + 4;         // LDS row stride in floats
  constexpr int LPR = W / 4;        // lanes per row (four columns each)
  constexpr int RPP = 64 / LPR;     // rows per pass
  const float alpha = p.g_a ? ld_uniform(p.g_a) * ld_uniform(p.g_w + e) : ld_uniform(p.g_w + e);
  const int ln = lane & 15, lg = lane >> 4;
  const int rr = lane / LPR, c4 = (lane % LPR) * 4;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i * 16 >= nrows) break;     // (uniform)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sh[(lg * 4 + r) * SW + 16 * j + ln] = alpha * acc[i][j][r];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int ps = 0; ps < 16 / RPP; ++ps) {
      const int row = i * 16 + ps * RPP + rr;
      const f32x4 v = *reinterpret_cast<const f32x4*>(sh + (ps * RPP + rr) * SW + c4);
      if (row < nrows) {
        const int64_t o = (int64_t)(row0 + row) * p.N + n_wave0 + c4;
        if constexpr (EPI == kEpiStoreF32) {
          *reinterpret_cast<f32x4*>(p.out_f32 + o) = v;
        } else {
          const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<u32x2*>(p.out_h + o) = u32x2{lo, hi};
        }
      }
    }
    // (the next m-tile rewrites sh only after every lane has read it)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Block-major epilogue of the SwiGLU GEMM1 variants for a wavefront's
// 16*MT rows x 16*NTW streaming columns (NTW/2 blocks of 16 h columns).  In
// the matrix-instruction layout a 16-element block of a row is spread over
// 16 lanes, so every lane would repeat the block's scale and bound
// computation for each of its values.  Instead the h values go through a
// wave-private LDS area sh ([16*MT][8*NTW] floats) and come back so that each
// lane owns whole blocks: one scale decision per block, and the codes, scale
// bytes and 16-bit copies leave as vector stores.
// Row stride (floats) of the h tile in LDS: 8 NTW columns plus 4 floats of
// padding, so that the four 4-row groups of a store and the 64-byte-apart
// block reads fall in different banks.
template <int NTW>
constexpr int kBlocksStride = 8 * NTW + 4;

template <int EPI, int MT, int NTW>
__device__ __forceinline__ void epilogue_blocks(const KParams& p, f32x4 (&acc)[MT][NTW], int e,
                                                int row0, int nrows, int n_wave0, int lane,
                                                float* __restrict__ sh) {
  static_assert(swiglu_epi(EPI), "SwiGLU epilogues only");
  constexpr int HC = 8 * NTW;                // h columns of the wave
  constexpr int SH = kBlocksStride<NTW>;     // LDS row stride (floats)
  constexpr int BLOCKS = 16 * MT * (HC / 16);
  static_assert(BLOCKS % kWave == 0, "whole blocks per lane");
  const float alpha = p.g_a ? ld_uniform(p.g_a) * ld_uniform(p.g_w + e) : ld_uniform(p.g_w + e);
  const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < NTW / 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gate = alpha * acc[i][2 * q][r];
        const float up = alpha * acc[i][2 * q + 1][r];
        sh[(i * 16 + lg * 4 + r) * SH + q * 16 + ln] = silu_fast(gate) * up;
      }
  // (wave-private area: the wave's own LDS writes are ordered before its reads)
  const int hb0 = n_wave0 >> 5;                // first 16-column block of h
  const float g2 = (EPI == kEpiSwigluFp4) ? ld_uniform(p.g2) : 0.0f;
#pragma unroll
  for (int j = 0; j < BLOCKS / kWave; ++j) {
    const int blk = lane + kWave * j;
    const int row = blk / (HC / 16), hb = blk % (HC / 16);
    const float* src = sh + row * SH + hb * 16;
    float v[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * w);
      v[4 * w] = x[0];
      v[4 * w + 1] = x[1];
      v[4 * w + 2] = x[2];
      v[4 * w + 3] = x[3];
    }
    if (row >= nrows) continue;
    const int64_t pr = row0 + row;
    if constexpr (EPI == kEpiSwigluFp4) {
      float am = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) am = fmaxf(am, fabsf(v[k]));
      const uint32_t sc = e4m3_scale_code(am, g2);
      const float sv = e4m3_value(sc);
      const E2M1Bounds bd = e2m1_bounds(sv, g2);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t code = e2m1_code(v[k], bd, sc == 0);
        if (k < 8) w0 |= code << (4 * k);
        else w1 |= code << (4 * (k - 8));
      }
      *reinterpret_cast<u32x2*>(p.out_q + pr * (p.I >> 1) + (hb0 + hb) * 8) = u32x2{w0, w1};
      p.out_sf[pr * (p.I >> 4) + hb0 + hb] = (uint8_t)sc;
      if (p.out_h) {
        // The exact f16 decoding of the 16 codes just written (the same
        // convert + scale multiply as the weights; exact, see dequant8_f16).
        const f16x2 s2 = f16x2_splat(sv);
        uint16_t* dst = p.out_h + pr * p.I + (hb0 + hb) * 16;
        *reinterpret_cast<f16x8*>(dst) = dequant8_f16(w0, s2);
        *reinterpret_cast<f16x8*>(dst + 8) = dequant8_f16(w1, s2);
      }
    } else {
      uint32_t bw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) bw[k] = f32_to_bf16_bits(v[2 * k]) | (f32_to_bf16_bits(v[2 * k + 1]) << 16);
      uint16_t* dst = p.out_h + pr * p.I + (hb0 + hb) * 16;
      *reinterpret_cast<u32x4*>(dst) = u32x4{bw[0], bw[1], bw[2], bw[3]};
      *reinterpret_cast<u32x4*>(dst + 8) = u32x4{bw[4], bw[5], bw[6], bw[7]};
    }
  }
}

// Row-group epilogue of the SwiGLU GEMM1 variants for short tiles (the
// streaming kernel), where often only a few of the 16 * MT rows are valid.
// In the matrix-instruction layout every lane holds 4 rows, so all four
// rounds of per-value work would run whatever the row count.  The h values go
// through a wave-private LDS area sh ([16*MT][2][8*NTW] floats: alpha-scaled
// gate and up) and come back with round t holding rows 4t..4t+3 (lane group
// g takes row 4t + g), so SwiGLU and the requantisation run only for the
// rounds up to the last valid row.  Each 16-lane row group then decides its
// block scale with a lane reduction, as in epilogue().
template <int EPI, int MT, int NTW>
__device__ __forceinline__ void epilogue_rows(const KParams& p, f32x4 (&acc)[MT][NTW], int e,
                                              int row0, int nrows, int n_wave0, int lane,
                                              float* __restrict__ sh) {
  static_assert(swiglu_epi(EPI), "SwiGLU epilogues only");
  constexpr int HC = 8 * NTW;                // h columns of the wave
  const float alpha = p.g_a ? ld_uniform(p.g_a) * ld_uniform(p.g_w + e) : ld_uniform(p.g_w + e);
  const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < NTW / 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = sh + (i * 16 + lg * 4 + r) * 2 * HC + q * 16 + ln;
        dst[0] = alpha * acc[i][2 * q][r];
        dst[HC] = alpha * acc[i][2 * q + 1][r];
      }
  // (wave-private area: the wave's own LDS writes are ordered before its reads)
  const int hb0 = n_wave0 >> 5;                // first 16-column block of h
  const float g2 = (EPI == kEpiSwigluFp4) ? ld_uniform(p.g2) : 0.0f;
  const int rounds = (min(nrows, 16 * MT) + 3) >> 2;
  for (int t = 0; t < rounds; ++t) {
    const int row = 4 * t + lg;
#pragma unroll
    for (int q = 0; q < NTW / 2; ++q) {
      const float* src = sh + row * 2 * HC + q * 16 + ln;
      const float h = silu_fast(src[0]) * src[HC];
      const int64_t pr = row0 + row;
      if constexpr (EPI == kEpiSwigluFp4) {
        const float am = row16_max(fabsf(h));
        const uint32_t sc = e4m3_scale_code(am, g2);
        const float sv = e4m3_value(sc);
        const E2M1Bounds bd = e2m1_bounds(sv, g2);
        const uint32_t code = e2m1_code(h, bd, sc == 0);
        const uint32_t other = (uint32_t)dpp_xor1_i((int)code);
        if (row < nrows) {
          if ((ln & 1) == 0)
            p.out_q[pr * (p.I >> 1) + (hb0 + q) * 8 + (ln >> 1)] = (uint8_t)(code | (other << 4));
          if (ln == 0) p.out_sf[pr * (p.I >> 4) + hb0 + q] = (uint8_t)sc;
          if (p.out_h) {
            // Exact: six significant bits at most, inside the f16 range.
            const float dv = e2m1_mag_value(code & 7u) * sv;
            const _Float16 hv = (_Float16)((code & 8u) ? -dv : dv);
            p.out_h[pr * p.I + (hb0 + q) * 16 + ln] = __builtin_bit_cast(uint16_t, hv);
          }
        }
      } else {
        if (row < nrows) p.out_h[pr * p.I + (hb0 + q) * 16 + ln] = (uint16_t)f32_to_bf16_bits(h);
      }
    }
  }
}

// Work item of a workgroup of the LDS kernel: (expert, first row, valid
// rows, column block).
struct Tile {
  int e, row0, nrows, nb;
};
// Tiles whose work shares data are kept on one XCD: the launch order is
// mapped so that each XCD receives a contiguous range of tiles.
__device__ __forceinline__ bool decode_tile(const KParams& p, Tile& t) {
  const int ntiles = ld_uniform(p.plan + p.list_idx);
  const int G = ntiles * p.n_blocks;
  if ((int)blockIdx.x >= G) return false;
  const int v = xcd_remap(blockIdx.x, G);
  const int tile = v / p.n_blocks;
  t.nb = v - tile * p.n_blocks;
  const int* ent = p.plan + ld_uniform(p.plan + kPlanLists + p.list_idx) + 2 * tile;
  t.e = ld_uniform(ent) & 2047;
  const uint32_t rr = (uint32_t)ld_uniform(ent + 1);
  t.row0 = (int)(rr & 0xFFFFFFu);
  t.nrows = (int)(rr >> 24);
  return true;
}

// Weight fragment of one 16x16x32 step as f16: 8 codes times the block scale
// of k-steps 0-1 (low half of s2) or 2-3 (high half).
__device__ __forceinline__ f16x8 weight_f16(uint32_t codes, f16x2 s2, int ks) {
  return dequant8_f16(codes, ks < 2 ? f16x2_lo(s2) : f16x2_hi(s2));
}

// ---------------------------------------------------------------------------
// LDS-staged kernel (tiles of 64 or 128 rows, the prefill regime).  A
// workgroup takes one tile and BN = NW * WN output columns.  Each wavefront
// owns WN columns for all BM rows: it streams its weight columns straight from
// HBM into registers while the BM x 128 activation chunk is staged once per
// workgroup in LDS (decoded to f16 for codes), double-buffered.
// ---------------------------------------------------------------------------
template <int AK, int EPI, int BM, int WN, int NW>
__global__ __launch_bounds__(NW * kWave) void grouped_gemm_kernel(KParams p) {
  constexpr int MT = BM / 16;
  constexpr int NTW = WN / 16;
  static_assert(NTW % 2 == 0, "scale words cover column tiles in pairs");
  // A staging pieces per chunk: 16-byte pieces of codes (32 elements) for
  // kActCodes, 16-byte pieces of 16-bit values (8 elements) otherwise.
  constexpr int PIECES = AK == kActCodes ? BM * 4 : BM * 16;
  static_assert(PIECES % (NW * kWave) == 0, "staging pieces split evenly over the threads");
  constexpr int PPT = PIECES / (NW * kWave);
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLDA];

  Tile t;
  if (!decode_tile(p, t)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_wave0 = (t.nb * NW + wv) * WN;
  const bool wave_on = n_wave0 < p.N;
  const int K = p.K, KC = K / kBK, NT = p.N / 16;

  // ---- A staging: each thread moves PPT pieces per chunk.  Rows past the
  // tile end repeat its last valid row (their results are never stored), so
  // every load is unconditional.
  const uint8_t* a_src[PPT];
  const uint8_t* s_src[PPT];
  int a_dst[PPT];  // element offset in a buffer
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int pc = tid + j * NW * kWave;
    const int r = AK == kActCodes ? (pc >> 2) : (pc >> 4);
    const int qq = AK == kActCodes ? (pc & 3) : (pc & 15);
    int src = t.row0 + min(r, t.nrows - 1);
    if (p.sorted_pair) src = pair_token(p.sorted_pair[src], p.T, p.topk);
    if constexpr (AK == kActCodes) {
      a_src[j] = p.a_q + (int64_t)src * (K >> 1) + qq * 16;
      s_src[j] = p.a_sf + (int64_t)src * (K >> 4) + qq * 2;
      a_dst[j] = r * kLDA + qq * 32;
    } else {
      a_src[j] = reinterpret_cast<const uint8_t*>(p.a_h + (int64_t)src * K + qq * 8);
      s_src[j] = nullptr;
      a_dst[j] = r * kLDA + qq * 8;
    }
  }
  u32x4 a_reg[PPT];
  uint32_t a_sreg[PPT];
  auto load_a = [&](int kc) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      if constexpr (AK == kActCodes) {
        a_reg[j] = *reinterpret_cast<const u32x4*>(a_src[j] + kc * 64);
        a_sreg[j] = *reinterpret_cast<const uint16_t*>(s_src[j] + kc * 8);
      } else {
        a_reg[j] = *reinterpret_cast<const u32x4*>(a_src[j] + kc * 256);
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      uint16_t* dst = &As[buf][a_dst[j]];
      if constexpr (AK == kActCodes) {
        const f16x2 s2 = e4m3x2_to_f16x2(a_sreg[j]);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<f16x8*>(dst + 8 * w) =
              dequant8_f16(a_reg[j][w], w < 2 ? f16x2_lo(s2) : f16x2_hi(s2));
      } else {
        *reinterpret_cast<u32x4*>(dst) = a_reg[j];
      }
    }
  };

  // ---- B (weights): this wave's column tiles, one 128-k chunk per load,
  // in two register sets used alternately.
  const int nt0 = n_wave0 >> 4;
  const int64_t wbase = ((int64_t)(t.e * NT + nt0) * KC) * kWave + lane;
  const uint8_t* s_expert = p.w_sf + (int64_t)t.e * (NT >> 1) * KC * 256;
  u32x4 bq0[NTW], bq1[NTW];
  uint32_t bs0[NTW / 2], bs1[NTW / 2];
  auto load_b = [&](int kc, u32x4 (&bq)[NTW], uint32_t (&bs)[NTW / 2]) {
    if (!wave_on) return;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
      bq[j] = *reinterpret_cast<const u32x4*>(p.w_q + (wbase + ((int64_t)j * KC + kc) * kWave) * 16);
#pragma unroll
    for (int j = 0; j < NTW / 2; ++j)
      bs[j] = *reinterpret_cast<const uint32_t*>(s_expert + scale_word_offset((nt0 >> 1) + j, kc, KC, lane));
  };

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int a_lrow = lane & 15, a_kq = (lane >> 4) * 32;
  auto compute = [&](int buf, const u32x4 (&bq)[NTW], const uint32_t (&bs)[NTW / 2]) {
    if (!wave_on) return;
    const uint16_t* abase = &As[buf][a_lrow * kLDA + a_kq];
    if constexpr (AK != kActBf16) {
      f16x2 sb2[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) sb2[j] = e4m3x2_to_f16x2(bs[j >> 1] >> ((j & 1) * 16));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bf[j] = weight_f16(bq[j][s], sb2[j], s);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const f16x8 af = *reinterpret_cast<const f16x8*>(abase + i * 16 * kLDA + 8 * s);
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    } else {
      float sb[NTW][2];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        // (hardware E4M3 -> f16, exact, then f16 -> f32, exact)
        const f16x2 h = e4m3x2_to_f16x2(bs[j >> 1] >> ((j & 1) * 16));
        sb[j][0] = (float)h[0];
        sb[j][1] = (float)h[1];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bf[j] = dequant8_bf16(bq[j][s], sb[j][s >> 1]);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(abase + i * 16 * kLDA + 8 * s);
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // ---- Pipeline: chunk kc computes from LDS buffer kc & 1 and register set
  // kc & 1 while chunk kc + 1 is in flight; one barrier per chunk.  A trip
  // runs two chunks so the register sets alternate statically; the
  // scheduling fences keep the next chunk's loads ahead of the compute.
  load_a(0);
  load_b(0, bq0, bs0);
  store_a(0);
  __syncthreads();
  // Every path back to the loop head passes the full wait (the exit tests
  // come after it), so the compiler knows no load is pending there.
  for (int kc = 0;; kc += 2) {
    const bool more1 = kc + 1 < KC;
    if (more1) {
      load_a(kc + 1);
      load_b(kc + 1, bq1, bs1);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(0, bq0, bs0);
    __builtin_amdgcn_sched_barrier(0);
    if (more1) store_a(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!more1) break;
    const bool more2 = kc + 2 < KC;
    if (more2) {
      load_a(kc + 2);
      load_b(kc + 2, bq0, bs0);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(1, bq1, bs1);
    __builtin_amdgcn_sched_barrier(0);
    if (more2) store_a(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!more2) break;
  }
  if (!wave_on) return;
  epilogue<EPI, MT, NTW>(p, acc, t.e, t.row0, t.nrows, n_wave0, lane);
}

// ---------------------------------------------------------------------------
// Wide kernel for 128-row tiles with 16-bit activations (the exact f16 copy
// of NVFP4 codes, or bf16 for W4A16): the prefill regime, bound by the
// matrix instructions and by weight decoding.  A workgroup computes 128 rows
// x 64 NW columns; each of its NW wavefronts owns 64 columns for all 128 rows,
// so every decoded weight fragment feeds 8 matrix instructions and every
// activation fragment read from LDS feeds 4; the activation chunk is brought
// in once for all NW wavefronts.  Activation chunks (128 rows x
// 128 k) move from memory to LDS with the direct-to-LDS loads of gfx950 (no
// registers, no VALU), double-buffered; the 16-byte units of a row are
// XOR-swizzled by the row so that the 16 rows of a fragment read fall in
// distinct banks.  Weights stream into two register sets used alternately.
// ---------------------------------------------------------------------------
#ifndef NVFP4_WIDE_INTERLEAVE
#define NVFP4_WIDE_INTERLEAVE 1  // interleave weight decode with matrix instructions
#endif
#ifndef NVFP4_WIDE_NW
#define NVFP4_WIDE_NW 4        // wavefronts per workgroup of the wide kernel (4 or 8)
#endif
#ifndef NVFP4_WIDE_WN
#define NVFP4_WIDE_WN 64       // columns per wavefront of the wide kernel (64 or 128)
#endif
// Waves per SIMD: 2 with 64 columns per wavefront, 1 with 128 (its 256
// accumulators take the accumulation registers).
#define NVFP4_WIDE_WPE (NVFP4_WIDE_WN == 128 ? 1 : 2)
#ifndef NVFP4_TALL_WN
#define NVFP4_TALL_WN 64       // columns per wavefront of the wide kernel for the tall experts of a split layer
#endif
// With f16 activations the wide kernel takes 32 columns per wavefront (twice
// the workgroups) where 64 would leave CU slots empty: both projections on
// 128-row tiles when the launch's bound on workgroups at 64 columns is at
// most NVFP4_SMALL_WIDE_GRID (the device holds 512 of them, two per CU), and
// the gate/up projection on the tall experts of a split layer.
#ifndef NVFP4_SMALL_WIDE_GRID
#define NVFP4_SMALL_WIDE_GRID 400
#endif
constexpr int kWideBM = 128, kWideWN = NVFP4_WIDE_WN, kWideNW = NVFP4_WIDE_NW;

template <int AK, int EPI, int WN>
__global__ __launch_bounds__(kWideNW * kWave)
__attribute__((amdgpu_waves_per_eu(NVFP4_WIDE_WPE, NVFP4_WIDE_WPE)))
void grouped_gemm_wide_kernel(KParams p) {
  static_assert(kWideNW == 4 || kWideNW == 8, "4 or 8 wavefronts");
  static_assert(AK != kActCodes, "the wide kernel takes 16-bit activations");
  static_assert(WN == 32 || WN == 64 || WN == 128, "whole tile pairs per wavefront");
  constexpr int MT = kWideBM / 16, NTW = WN / 16, NW = kWideNW;
  constexpr int ROW_BYTES = kBK * 2;                       // 256
  constexpr int BUF_BYTES = kWideBM * ROW_BYTES;           // 32 KiB
  constexpr int LOADS = BUF_BYTES / (NW * kWave * 16);     // direct loads per thread per chunk: 8
  // Two separate arrays (not one array of two halves): the compiler can then
  // tell that reads of one buffer do not alias the direct loads filling the
  // other, and does not drain the loads before every read.
  __shared__ __attribute__((aligned(16))) uint8_t As0[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As1[BUF_BYTES];

  Tile t;
  if (!decode_tile(p, t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_wave0 = (t.nb * NW + wv) * WN;
  const bool wave_on = n_wave0 < p.N;
  const int K = p.K, KC = K / kBK, NT = p.N / 16;

  // ---- B (weights), two register sets.
  const int nt0 = n_wave0 >> 4;
  const int64_t wbase = ((int64_t)(t.e * NT + nt0) * KC) * kWave + lane;
  const uint8_t* s_expert = p.w_sf + (int64_t)t.e * (NT >> 1) * KC * 256;
  u32x4 bq0[NTW], bq1[NTW];
  uint32_t bs0[NTW / 2], bs1[NTW / 2];
  auto load_b = [&](int kc, u32x4 (&bq)[NTW], uint32_t (&bs)[NTW / 2]) {
    if (!wave_on) return;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
      bq[j] = *reinterpret_cast<const u32x4*>(p.w_q + (wbase + ((int64_t)j * KC + kc) * kWave) * 16);
#pragma unroll
    for (int j = 0; j < NTW / 2; ++j)
      bs[j] = *reinterpret_cast<const uint32_t*>(s_expert + scale_word_offset((nt0 >> 1) + j, kc, KC, lane));
  };
  // The weights of chunk 0 do not depend on the activation rows: they are
  // requested first, so their latency overlaps the sorted-pair gather.
  load_b(0, bq0, bs0);

  // ---- A staging.  Load q of wave wv fills LDS bytes [(wv*LOADS+q) KiB, +1 KiB)
  // of a buffer: rows 4(wv*LOADS+q) + lane/16, LDS unit lane%16, which holds
  // source unit (lane%16) ^ (row%16) of the row.  Rows past the tile end
  // repeat its last valid row (their results are never stored).
  uint32_t a_off[LOADS];
  int src[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) src[q] = t.row0 + min(4 * (wv * LOADS + q) + (lane >> 4), t.nrows - 1);
  if (p.sorted_pair) {
    int f[LOADS];  // all gathers in flight together
#pragma unroll
    for (int q = 0; q < LOADS; ++q) f[q] = p.sorted_pair[src[q]];
#pragma unroll
    for (int q = 0; q < LOADS; ++q) src[q] = pair_token(f[q], p.T, p.topk);
  }
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int r = 4 * (wv * LOADS + q) + (lane >> 4);
    const int unit = (lane & 15) ^ (r & 15);
    a_off[q] = (uint32_t)src[q] * (uint32_t)(K * 2) + (uint32_t)unit * 16u;
  }
  const uint8_t* a_base = reinterpret_cast<const uint8_t*>(p.a_h);
  // The direct loads are issued as assembly: the compiler treats a
  // direct-to-LDS load as a pending write that any later LDS read may alias
  // and drains the load counter before every read, which would serialise the
  // prefetch of chunk kc + 1 with the compute of chunk kc.  Completion is
  // awaited explicitly (lds_fill_wait) before the barrier that publishes a
  // buffer.
  auto stage_a = [&, a_base](auto mta, int kc, uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      if (4 * (wv * LOADS + q) >= 16 * decltype(mta)::value) continue;  // rows no m-tile reads
      const uint32_t lds = (uint32_t)(uintptr_t)(buf + (wv * LOADS + q) * 1024);
      const uint32_t voff = a_off[q] + (uint32_t)kc * ROW_BYTES;
      asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(a_base), "{m0}"(lds) : "memory");
    }
  };
  // (builtin, not assembly: the compiler must see that every load, its own
  // included, has completed, or it re-waits before reusing load registers)
  auto lds_fill_wait = [] { __builtin_amdgcn_s_waitcnt(0); };

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragment read: lane (m = lane%16, g = lane/16) takes row i*16 + m, k in
  // [32g + 8s, 32g + 8s + 8), i.e. source unit 4g + s, stored at unit
  // (4g + s) ^ m of the row.
  const int m = lane & 15, g = lane >> 4;
  auto compute = [&](auto mta, const uint8_t* buf, const u32x4 (&bq)[NTW], const uint32_t (&bs)[NTW / 2]) __attribute__((always_inline)) {
    constexpr int MA = decltype(mta)::value;  // m-tiles holding rows of this tile
    if (!wave_on) return;
    const uint8_t* abuf = buf + m * ROW_BYTES;
    if constexpr (AK == kActF16) {
      f16x2 sb2[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) sb2[j] = e4m3x2_to_f16x2(bs[j >> 1] >> ((j & 1) * 16));
      // Per k-step: all fragment reads first; then column tile by column
      // tile, the decode of tile j + 1 (8 VALU instructions) is interleaved
      // with the 8 matrix instructions of tile j, so it issues while the
      // matrix unit is busy.
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ucol = ((4 * g + s) ^ m) * 16;
        f16x8 af[MA];
#pragma unroll
        for (int i = 0; i < MA; ++i) af[i] = *reinterpret_cast<const f16x8*>(abuf + i * 16 * ROW_BYTES + ucol);
        __builtin_amdgcn_sched_barrier(0);
        f16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bf[j] = weight_f16(bq[j][s], sb2[j], s);
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int i = 0; i < MA; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
#if NVFP4_WIDE_INTERLEAVE
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // decode of tile 0
#pragma unroll
        for (int j = 0; j + 1 < NTW; ++j)
#pragma unroll
          for (int i = 0; i < MA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // one decode instruction
          }
        __builtin_amdgcn_sched_group_barrier(0x008, MA, 0);  // the last tile's
#endif
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      float sb[NTW][2];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        // (hardware E4M3 -> f16, exact, then f16 -> f32, exact)
        const f16x2 h = e4m3x2_to_f16x2(bs[j >> 1] >> ((j & 1) * 16));
        sb[j][0] = (float)h[0];
        sb[j][1] = (float)h[1];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ucol = ((4 * g + s) ^ m) * 16;
        bf16x8 af[MA];
#pragma unroll
        for (int i = 0; i < MA; ++i) af[i] = *reinterpret_cast<const bf16x8*>(abuf + i * 16 * ROW_BYTES + ucol);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bf[j] = dequant8_bf16(bq[j][s], sb[j][s >> 1]);
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int i = 0; i < MA; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
#if NVFP4_WIDE_INTERLEAVE
        // (the bf16 decode of a tile is 16 VALU instructions: two per matrix
        // instruction of the previous tile)
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
#pragma unroll
        for (int j = 0; j + 1 < NTW; ++j)
#pragma unroll
          for (int i = 0; i < MA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
        __builtin_amdgcn_sched_group_barrier(0x008, MA, 0);
#endif
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- Pipeline (as in the LDS-staged kernel): chunk kc computes from LDS
  // buffer kc & 1 and register set kc & 1 while chunk kc + 1 lands; the
  // direct loads are complete once the vector counter drains, then one
  // barrier per chunk publishes the buffer.
  auto main_loop = [&](auto mta) __attribute__((always_inline)) {
    stage_a(mta, 0, As0);
    lds_fill_wait();
    __syncthreads();
    // Every path back to the loop head passes the full wait (the exit tests
    // come after it), so the compiler knows no load is pending there and does
    // not drain the counter before the next refills.
    for (int kc = 0;; kc += 2) {
      const bool more1 = kc + 1 < KC;
      if (more1) {
        stage_a(mta, kc + 1, As1);
        load_b(kc + 1, bq1, bs1);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(mta, As0, bq0, bs0);
      __builtin_amdgcn_sched_barrier(0);
      lds_fill_wait();
      __syncthreads();
      if (!more1) break;
      const bool more2 = kc + 2 < KC;
      if (more2) {
        stage_a(mta, kc + 2, As0);
        load_b(kc + 2, bq0, bs0);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(mta, As1, bq1, bs1);
      __builtin_amdgcn_sched_barrier(0);
      lds_fill_wait();
      __syncthreads();
      if (!more2) break;
    }
  };
  // The last tile of an expert is usually short: only the m-tiles that hold
  // its rows are staged and multiplied (the weight stream and decode are the
  // same for every tile height).  The choice is uniform over the workgroup.
  const int mt_rows = (t.nrows + 15) >> 4;
  if (mt_rows > MT / 2) main_loop(std::integral_constant<int, MT>{});
  else if (mt_rows > MT / 4) main_loop(std::integral_constant<int, MT / 2>{});
  else if (mt_rows > 1) main_loop(std::integral_constant<int, MT / 4>{});
  else main_loop(std::integral_constant<int, 1>{});
  if (!wave_on) return;
  // The activation buffers are free (the loop ended on a barrier after the
  // last reads): each wavefront takes 1/NW of them for its epilogue.
  constexpr int WAVE_BYTES = 2 * BUF_BYTES / NW;
  uint8_t* const area = (wv < NW / 2 ? As0 : As1) + (wv % (NW / 2)) * WAVE_BYTES;
  float* sh = reinterpret_cast<float*>(area);
  if constexpr (!swiglu_epi(EPI)) {
    static_assert(16 * (16 * NTW + 4) * 4 <= WAVE_BYTES, "one m-tile fits the wave's area");
    epilogue_rowmajor<EPI, MT, NTW>(p, acc, t.e, t.row0, t.nrows, n_wave0, lane, sh);
  } else {
    // SwiGLU: passes of PM m-tiles (4 with 4 wavefronts, 2 with 8).
    constexpr int PMF = WAVE_BYTES / (16 * kBlocksStride<NTW> * 4);
    constexpr int PM = PMF >= 8 ? 8 : PMF >= 4 ? 4 : PMF >= 2 ? 2 : 1;
    static_assert(PM >= 1 && MT % PM == 0, "whole m-tiles per pass");
#pragma unroll
    for (int pm = 0; pm < MT; pm += PM)
      epilogue_blocks<EPI, PM, NTW>(p, *reinterpret_cast<f32x4(*)[PM][NTW]>(&acc[pm]), t.e,
                                    t.row0 + pm * 16, t.nrows - pm * 16, n_wave0, lane, sh);
  }
}

// ---------------------------------------------------------------------------
// Persistent streaming kernel for short tiles (16 or 32 rows), the decode
// regime where every weight byte is read once and the time is the weight
// stream.  Work units are (tile, group of NTW column tiles); wavefront w of
// W resident ones takes units w, w + W, w + 2W, ... (a fixed, deterministic
// assignment).  Each wavefront keeps a ring of PF 128-k chunks in flight and
// the ring does not drain between units: the last round of a unit refills
// the slots with the first chunks of the wavefront's next unit.  Activation
// fragments ride in the ring beside the weights, in the weights' lane layout
// (lane 16g + m holds row m, k in [32g, 32g + 32) of a chunk).
//
// NVFP4 codes are decoded by every wavefront that uses them.  16-bit
// activations (the exact f16 copy, or bf16) need no decoding, and the four
// wavefronts of a workgroup always work on the same tile (the unit count per
// tile and the wavefront stride are multiples of four): each loads four of
// the tile's 16 rows of the chunk (256 contiguous bytes per row, so every
// load is coalesced), stores them in LDS, and after one barrier all four read
// their fragments from there.  The LDS fence covers LDS only, so the barrier
// never waits for the weight ring.
// ---------------------------------------------------------------------------
// Scale words of G consecutive chunks (4G contiguous bytes per lane).
template <int G>
struct ScaleGroup {
  uint32_t w[G];
  __device__ __forceinline__ static ScaleGroup load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    ScaleGroup s;
    if constexpr (G == 4) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
      s.w[0] = v[0]; s.w[1] = v[1]; s.w[2] = v[2]; s.w[3] = v[3];
    } else if constexpr (G == 3) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
      s.w[0] = v[0]; s.w[1] = v[1]; s.w[2] = v[2];
    } else if constexpr (G == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
      s.w[0] = v[0]; s.w[1] = v[1];
    } else {
      s.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    return s;
  }
};

template <int AK, int EPI, int MT, int NTW, int PF>
__device__ __forceinline__ void stream_body(const KParams& p) {
  static_assert(NTW % 2 == 0, "scale words cover column tiles in pairs");
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kNW + (threadIdx.x >> 6)));
  const int K = p.K, KC = K / kBK, NT = p.N / 16, CG = NT / NTW;
  const int n_units = ld_uniform(p.plan + p.list_idx) * CG;
  if (n_units == 0) return;
  // The launch covers the largest possible plan; every launched wavefront
  // takes units while there are any (wavefront w: units w, w + W, ...), so
  // some take one more unit than others.  Measured at decode (6144 units,
  // 4096 wavefronts): 47.3 us, against 49.1 us when only 3072 wavefronts
  // took two units each -- more loads in flight in the first round outweigh
  // the half-occupied second one.  W is a multiple of 4 (whole workgroups),
  // and so is the unit count per tile when activations are shared.
  constexpr bool COOP = AK != kActCodes;
  const int W_launch = gridDim.x * kNW;
  const int W = min(W_launch, n_units);
  if (wave >= W) return;
  const int* list = p.plan + ld_uniform(p.plan + kPlanLists + p.list_idx);
  const int wq = threadIdx.x >> 6;  // COOP: the 32-k step this wavefront loads

  // Buffer addressing: a scalar descriptor per operand (per expert for the
  // weights) plus a 32-bit per-lane offset; every byte range addressed here
  // is below 2^31 (checked by the launcher).
  const int64_t wq_expert = (int64_t)NT * KC * 1024;  // code bytes per expert
  const int64_t ws_expert = (int64_t)(NT >> 1) * KC * 256;
  // The ring holds one group of PF chunks: the weight scales of a tile pair
  // for the whole group arrive with one load per lane.
  static_assert(PF >= 1 && PF <= 4, "ring depth = scale group");
  const int w_lane = lane * 16, s_lane = lane * 4 * PF;
  const __amdgpu_buffer_rsrc_t a_rsrc = AK == kActCodes
      ? __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, (short)0, 0x7FFFFFFF, kBufferFlags)
      : __builtin_amdgcn_make_buffer_rsrc((void*)p.a_h, (short)0, 0x7FFFFFFF, kBufferFlags);
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(AK == kActCodes ? p.a_sf : p.w_sf), (short)0, 0x7FFFFFFF, kBufferFlags);

  // Work unit: expert, rows, first column, and the per-lane activation row
  // offsets (rows past the tile end repeat its last valid row; their results
  // are never stored).
  struct Unit {
    int e, row0, nrows, n0, nt0;
    int a_off[MT], s_off[MT];
  };
  auto unit = [&](int u) {
    Unit U;
    const int tile = u / CG, cg = u - tile * CG;
    U.e = ld_uniform(list + 2 * tile) & 2047;
    const uint32_t rr = (uint32_t)ld_uniform(list + 2 * tile + 1);
    U.row0 = (int)(rr & 0xFFFFFFu);
    U.nrows = (int)(rr >> 24);
    U.nt0 = cg * NTW;
    U.n0 = U.nt0 * 16;
    // Row of the tile this lane loads: its fragment row, or (COOP) row
    // 4 * wq + lane / 16 with lane % 16 selecting the 16-byte piece.
    const int rl = COOP ? 4 * wq + (lane >> 4) : (lane & 15);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      int r = U.row0 + min(i * 16 + rl, U.nrows - 1);
      if (p.sorted_pair) {
        // The 16 pair indices of this m-tile through scalar loads, then each
        // lane picks its own (a vector gather here would be waited for with
        // the in-order vector counter, i.e. behind the whole ring).
        int f = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int fq = ld_uniform(p.sorted_pair + U.row0 + min(i * 16 + q, U.nrows - 1));
          f = rl == q ? fq : f;
        }
        r = pair_token(f, p.T, p.topk);
      }
      U.a_off[i] = AK == kActCodes ? r * (K >> 1) + g * 16 : r * K * 2 + (lane & 15) * 16;
      U.s_off[i] = r * (K >> 4) + g * 2;
    }
    return U;
  };

  u32x4 bq[PF][NTW];
  // Scale words of the group being computed (bs) and of the next one (bsn,
  // loaded with the group's first refill).
  ScaleGroup<PF> bs[NTW / 2], bsn[NTW / 2];
  // 16-byte activation words per m-tile and chunk held by this wavefront.
  constexpr int AW = (AK == kActCodes || COOP) ? 1 : 4;
  u32x4 aq[PF][MT][AW];
  // COOP: [2 buffers][16 MT rows][272 bytes] (a 256-byte chunk row plus 16
  // bytes of padding, which spreads the fragment reads over all banks), one
  // buffer per chunk.
  constexpr int kRowB = 272, kBufB = 16 * MT * kRowB;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[COOP ? 2 * kBufB : 16];
  int abuf = 0;
  uint32_t as[PF][MT];
  // Refill of ring slot ``slot`` with chunk kc of unit A (sel false) or B
  // (sel true).  The choice is made with selects, not a branch: the loads
  // must be unconditional for the hardware load counter to be tracked
  // exactly (a branch makes the compiler wait for the whole ring).
  auto load = [&](const Unit& A, const Unit& B, bool sel, int kc, int slot) {
    const int e = sel ? B.e : A.e, nt0 = sel ? B.nt0 : A.nt0;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w_q + e * wq_expert), (short)0, 0x7FFFFFFF, kBufferFlags);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w_sf + e * ws_expert), (short)0, 0x7FFFFFFF, kBufferFlags);
#pragma unroll
    for (int j = 0; j < NTW; ++j)
      bq[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, w_lane, ((nt0 + j) * KC + kc) * 1024, 0));
    if (slot == 0) {
#pragma unroll
      for (int j = 0; j < NTW / 2; ++j)
        bsn[j] = ScaleGroup<PF>::load(sr, s_lane, (((nt0 >> 1) + j) * (KC / PF) + kc / PF) * 256 * PF);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int ao = sel ? B.a_off[i] : A.a_off[i];
      if constexpr (AK == kActCodes) {
        const int so = sel ? B.s_off[i] : A.s_off[i];
        aq[slot][i][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, ao, kc * 64, 0));
        as[slot][i] = __builtin_amdgcn_raw_buffer_load_b16(as_rsrc, so, kc * 8, 0);
      } else {
#pragma unroll
        for (int w = 0; w < AW; ++w)
          aq[slot][i][w] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, ao + w * 16, kc * 256, 0));
      }
    }
  };
  // COOP: publish this wavefront's k-step of the chunk in slot ``slot`` and
  // return once all four are readable.  Double-buffered: a buffer is written
  // again two chunks later, after every wavefront has passed the barrier that
  // follows its reads (the fence before each barrier completes them).
  auto share_a = [&](int slot) {
    uint8_t* buf = a_lds + abuf * kBufB;
#pragma unroll
    for (int i = 0; i < MT; ++i)
      *reinterpret_cast<u32x4*>(buf + (i * 16 + 4 * wq + (lane >> 4)) * kRowB + (lane & 15) * 16) =
          aq[slot][i][0];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // Fragment of k-step ks: row lane % 16, k in [32 g + 8 ks, 32 g + 8 ks + 8)
  // (the k order of the weight fragments).
  auto shared_a = [&](int i, int ks) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(a_lds + abuf * kBufB + (i * 16 + (lane & 15)) * kRowB +
                                           g * 64 + ks * 16);
  };

  // SwiGLU epilogues: a wave-private h tile in LDS.
  __shared__ float h_lds[swiglu_epi(EPI) ? kNW * 16 * MT * 16 * NTW : 1];
  float* const sh = h_lds + (swiglu_epi(EPI) ? wq * 16 * MT * 16 * NTW : 0);

  f32x4 acc[MT][NTW];
  auto compute = [&](int slot) {
    if constexpr (COOP) share_a(slot);
    if constexpr (AK != kActBf16) {
      f16x2 sa2[MT], sb2[NTW];
      if constexpr (AK == kActCodes) {
#pragma unroll
        for (int i = 0; i < MT; ++i) sa2[i] = e4m3x2_to_f16x2(as[slot][i]);
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j) sb2[j] = e4m3x2_to_f16x2(bs[j >> 1].w[slot] >> ((j & 1) * 16));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        f16x8 af[MT], bf[NTW];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if constexpr (AK == kActCodes)
            af[i] = dequant8_f16(aq[slot][i][0][ks], ks < 2 ? f16x2_lo(sa2[i]) : f16x2_hi(sa2[i]));
          else
            af[i] = __builtin_bit_cast(f16x8, shared_a(i, ks));
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) bf[j] = weight_f16(bq[slot][j][ks], sb2[j], ks);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    } else {
      float sb[NTW][2];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const f16x2 h = e4m3x2_to_f16x2(bs[j >> 1].w[slot] >> ((j & 1) * 16));
        sb[j][0] = (float)h[0];
        sb[j][1] = (float)h[1];
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bf[j] = dequant8_bf16(bq[slot][j][ks], sb[j][ks >> 1]);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, shared_a(i, ks));
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // The unit after a wave's last one points its weight loads at the first
  // chunks of expert 0's first column tiles, which every wave reads, so those
  // (unused) refills stay in L2 and every load remains unconditional.
  auto next_unit = [&](int u_next, bool more) {
    Unit n = unit(more ? u_next : u_next - W);
    n.e = more ? n.e : 0;
    n.nt0 = more ? n.nt0 : 0;
    return n;
  };
  int u = wave;
  Unit cur = unit(u);
  bool more = u + W < n_units;
  Unit nxt = next_unit(u + W, more);
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    load(cur, cur, false, s, s);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < NTW / 2; ++j) bs[j] = bsn[j];
  while (true) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kc0 = 0; kc0 < KC; kc0 += PF) {
      const bool last_round = kc0 + PF >= KC;
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        compute(s);
        abuf ^= 1;
        __builtin_amdgcn_sched_barrier(0);
        // PF divides KC, so the next unit's chunk index is s.
        load(cur, nxt, last_round, last_round ? s : kc0 + PF + s, s);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The next group's scales were requested before its weights, so this
      // waits for nothing that the next compute would not wait for anyway.
#pragma unroll
      for (int j = 0; j < NTW / 2; ++j) bs[j] = bsn[j];
    }
    if constexpr (!swiglu_epi(EPI))
      epilogue<EPI, MT, NTW>(p, acc, cur.e, cur.row0, cur.nrows, cur.n0, lane);
    else
      epilogue_rows<EPI, MT, NTW>(p, acc, cur.e, cur.row0, cur.nrows, cur.n0, lane, sh);
    if (!more) break;
    u += W;
    cur = nxt;
    more = u + W < n_units;
    nxt = next_unit(u + W, more);
  }
  // Let the final (unused) refills land before the wave ends.
  __builtin_amdgcn_s_waitcnt(0);
}

// Register budget: instantiations whose ring fits in 128 registers run 4
// wavefronts per SIMD (more weight bytes in flight per CU); the others are
// left to the compiler (a forced budget would spill).
template <int AK, int MT, int PF>
constexpr bool stream_fits_four_waves() {
  return MT == 1 || PF <= 3;
}

template <int AK, int EPI, int MT, int NTW, int PF>
__global__ __launch_bounds__(kNW * kWave) void grouped_gemm_stream_kernel(KParams p) {
  stream_body<AK, EPI, MT, NTW, PF>(p);
}

template <int AK, int EPI, int MT, int NTW, int PF>
__global__ __launch_bounds__(kNW * kWave) __attribute__((amdgpu_waves_per_eu(4, 8)))
void grouped_gemm_stream4_kernel(KParams p) {
  stream_body<AK, EPI, MT, NTW, PF>(p);
}

// out[t] = sum_j w[t][j] * d[inv_pos[t*k + j]] (+ shared row), FP32, j ascending.
// NT: read the rows with non-temporal loads (for workspaces larger than the
// caches; a small workspace, still cached from GEMM2, is read faster with
// ordinary loads).
template <bool BF16, bool NT>
__device__ __forceinline__ f32x4 load_row4(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  else return *reinterpret_cast<const f32x4*>(p);
}

template <bool BF16, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ d,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int topk, int shared, int H, void* out) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= H) return;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  // Batches of 8 pairs: positions and weights (the same for the whole block)
  // through scalar loads, then all 8 row loads in flight together, then the
  // sum in ascending j (selects, not branches, so no load waits on another).
  constexpr int B = 8;
  for (int j0 = 0; j0 < topk; j0 += B) {
    int pos[B];
    float w[B];
    f32x4 x[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int j = j0 + b;
      pos[b] = j < topk ? ld_uniform(inv_pos + (int64_t)t * topk + j) : -1;
      w[b] = j < topk ? ld_uniform(topk_w + (int64_t)t * topk + j) : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) x[b] = load_row4<BF16, NT>(d + (int64_t)max(pos[b], 0) * H + c);
#pragma unroll
    for (int b = 0; b < B; ++b) a = pos[b] >= 0 ? a + w[b] * x[b] : a;
  }
  if (shared) {
    const int pos = inv_pos[(int64_t)T * topk + t];
    if (pos >= 0) a += load_row4<BF16, NT>(d + (int64_t)pos * H + c);
  }
  if constexpr (BF16) {
    uint32_t lo = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
    uint32_t hi = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + (int64_t)t * H + c) = u32x2{lo, hi};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)t * H + c) = a;
  }
}

// ---------------------------------------------------------------------------
// Dense linear layer for at most 16 rows (the decode shape of a dense
// layer): one workgroup per 2 column tiles (32 columns), its 4 wavefronts
// splitting K into quarters, each loading UB chunks (weights, activation
// codes or bf16 values, scales) before decoding and multiplying them;
// the partial sums meet in LDS in a fixed order.  Four times the wavefronts
// of a persistent pass over (tile, 32-column) units, which at N = 34816
// leaves most of the device idle for a single 16-row tile.
// ---------------------------------------------------------------------------
template <int AK, bool F32, int UB>
__global__ __launch_bounds__(4 * kWave) void linear_splitk_kernel(KParams p) {
  constexpr int NTW = 2;
  static_assert(AK != kActF16, "codes or bf16 activations");
  __shared__ f32x4 red[3][NTW][kWave];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int M = p.T, N = p.N, K = p.K, KC = K / kBK, NT = N / 16;
  const int c_lo = KC * wv / 4, c_hi = KC * (wv + 1) / 4;
  const int nt0 = blockIdx.x * NTW;
  const int row = min(m, M - 1);   // rows past M repeat the last one (never stored)
  f32x4 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = c_lo; c0 < c_hi; c0 += UB) {
    u32x4 bq[UB][NTW];
    uint32_t bs[UB];
    u32x4 aq[UB][AK == kActCodes ? 1 : 4];
    uint32_t as[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int kc = min(c0 + u, c_hi - 1);   // a repeated chunk is loaded but not used
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        bq[u][j] = *reinterpret_cast<const u32x4*>(p.w_q + ((int64_t)((nt0 + j) * KC + kc) * kWave + lane) * 16);
      bs[u] = *reinterpret_cast<const uint32_t*>(p.w_sf + scale_word_offset(nt0 >> 1, kc, KC, lane));
      if constexpr (AK == kActCodes) {
        aq[u][0] = *reinterpret_cast<const u32x4*>(p.a_q + (int64_t)row * (K / 2) + kc * 64 + g * 16);
        as[u] = *reinterpret_cast<const uint16_t*>(p.a_sf + (int64_t)row * (K / 16) + kc * 8 + g * 2);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          aq[u][w] = *reinterpret_cast<const u32x4*>(p.a_h + (int64_t)row * K + kc * kBK + g * 32 + w * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (c0 + u >= c_hi) continue;
      if constexpr (AK == kActCodes) {
        const f16x2 sa2 = e4m3x2_to_f16x2(as[u]);
        f16x2 sb2[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) sb2[j] = e4m3x2_to_f16x2(bs[u] >> (j * 16));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f16x8 af = dequant8_f16(aq[u][0][ks], ks < 2 ? f16x2_lo(sa2) : f16x2_hi(sa2));
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, weight_f16(bq[u][j][ks], sb2[j], ks), acc[j], 0, 0, 0);
        }
      } else {
        float sb[NTW][2];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const f16x2 h = e4m3x2_to_f16x2(bs[u] >> (j * 16));
          sb[j][0] = (float)h[0];
          sb[j][1] = (float)h[1];
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, aq[u][ks]);
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, dequant8_bf16(bq[u][j][ks], sb[j][ks >> 1]),
                                                             acc[j], 0, 0, 0);
        }
      }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) red[wv - 1][j][lane] = acc[j];
  }
  __syncthreads();
  if (wv > 0) return;
  const float alpha = p.g_a ? ld_uniform(p.g_a) * ld_uniform(p.g_w) : ld_uniform(p.g_w);
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    f32x4 v = acc[j];
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const f32x4 o = red[w][j][lane];
      v[0] += o[0];
      v[1] += o[1];
      v[2] += o[2];
      v[3] += o[3];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = g * 4 + r;
      if (rr < M) {
        const int64_t o = (int64_t)rr * N + (nt0 + j) * 16 + m;
        if constexpr (F32) p.out_f32[o] = alpha * v[r];
        else p.out_h[o] = (uint16_t)f32_to_bf16_bits(alpha * v[r]);
      }
    }
  }
  (void)NT;
}


template <int AK, int EPI, int WN = kWideWN>
hipError_t launch_wide(KParams kp, int list_len, hipStream_t s) {
  kp.n_blocks = (kp.N + kWideNW * WN - 1) / (kWideNW * WN);
  const int64_t G = (int64_t)list_len * kp.n_blocks;
  const int64_t grid = std::max<int64_t>(8, (G + 7) / 8 * 8);
  grouped_gemm_wide_kernel<AK, EPI, WN><<<(unsigned)grid, kWideNW * kWave, 0, s>>>(kp);
  return hipGetLastError();
}

template <int AK, int EPI, int BM, int WN>
hipError_t launch_lds(KParams kp, int list_len, hipStream_t s) {
  constexpr int NW = NVFP4_BIG_NW;
  kp.n_blocks = (kp.N + NW * WN - 1) / (NW * WN);
  const int64_t G = (int64_t)list_len * kp.n_blocks;
  const int64_t grid = std::max<int64_t>(8, (G + 7) / 8 * 8);
  grouped_gemm_kernel<AK, EPI, BM, WN, NW><<<(unsigned)grid, NW * kWave, 0, s>>>(kp);
  return hipGetLastError();
}

// Persistent launch: as many workgroups as fit on the device at once (the
// occupancy of this kernel times the CU count), capped by the work.  Both
// figures are queried on every call (host-side lookups), so nothing is kept
// between calls and each device answers for itself.
template <auto KERN>
hipError_t launch_persistent(const KParams& kp, int64_t units, hipStream_t s) {
  int nb = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(KERN),
                                                              kNW * kWave, 0);
  if (e != hipSuccess) return e;
  const int per_cu = nb > 0 ? nb : 1;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t need = (units + kNW - 1) / kNW;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((int64_t)per_cu * cus, need));
  KERN<<<(unsigned)grid, kNW * kWave, 0, s>>>(kp);
  return hipGetLastError();
}

template <int AK, int EPI, int MT, int NTW, int PF>
hipError_t launch_stream(const KParams& kp, int list_len, hipStream_t s) {
  const int64_t cg = (kp.N / 16) / NTW;
  // 16-bit activations are shared by the workgroup's four wavefronts, which
  // must all work on one tile: the units per tile come in fours.
  if (AK != kActCodes && cg % kNW != 0) return hipErrorInvalidValue;
  const int64_t units = (int64_t)list_len * cg;
  if constexpr (stream_fits_four_waves<AK, MT, PF>())
    return launch_persistent<grouped_gemm_stream4_kernel<AK, EPI, MT, NTW, PF>>(kp, units, s);
  else
    return launch_persistent<grouped_gemm_stream_kernel<AK, EPI, MT, NTW, PF>>(kp, units, s);
}

// Ring depth of the streaming kernel: one scale group of the weights.
template <int AK, int EPI, int MT, int NTW>
hipError_t launch_stream_pf(const KParams& kp, int len, hipStream_t s) {
  switch (scale_group(kp.K / kBK)) {
    case 4: return launch_stream<AK, EPI, MT, NTW, 4>(kp, len, s);
    case 3: return launch_stream<AK, EPI, MT, NTW, 3>(kp, len, s);
    case 2: return launch_stream<AK, EPI, MT, NTW, 2>(kp, len, s);
    default: return launch_stream<AK, EPI, MT, NTW, 1>(kp, len, s);
  }
}

// part (kPart*): kPartShort and kPartTall launch one list each of a split
// layer; a layer that is not split runs whole under kPartShort and not at
// all under kPartTall, so the two always add up to kPartAll.
template <int AK, int EPI>
hipError_t launch_gemm(KParams kp, const AlignShape& al, hipStream_t s, int part) {
  constexpr int kStreamNTW = swiglu_epi(EPI) ? NVFP4_STREAM_NTW : NVFP4_STREAM_NTW_DOWN;
  int li = min(pick_list(al.P, al.slots), NVFP4_LIST_MAX);
  // The streaming kernel addresses with 32-bit buffer offsets.
  const int64_t a_row_bytes = AK == kActCodes ? kp.K / 2 : 2 * (int64_t)kp.K;
  const bool offsets_fit = kp.a_rows * a_row_bytes < (int64_t(1) << 31) &&
                           (int64_t)kp.N * kp.K / 2 < (int64_t(1) << 31);
  if (li <= 1 && !offsets_fit) li = 2;
  if constexpr (AK != kActCodes) {
    // 16-bit activations on tall tiles: the wide kernel (128-row tiles).
    constexpr bool kUp32 = swiglu_epi(EPI) && AK == kActF16;
    if (li >= NVFP4_WIDE_MIN_LIST && offsets_fit) {
      if (part == kPartTall) return hipSuccess;
      kp.list_idx = 3;
      if constexpr (AK == kActF16) {
        if (al.list_len[3] * ((kp.N + 255) / 256) <= NVFP4_SMALL_WIDE_GRID)
          return launch_wide<AK, EPI, 32>(kp, (int)al.list_len[3], s);
      }
      return launch_wide<AK, EPI>(kp, (int)al.list_len[3], s);
    }
    // Short tiles on average, but some experts may hold many rows: the
    // streaming kernel would read their weights once per 16-row tile, so
    // those experts (list 5) go to the wide kernel and the rest (list 4) to
    // the streaming kernel.  Two launches writing disjoint rows.
    if (split_experts(al) && offsets_fit) {
      if (part != kPartTall) {
        kp.list_idx = 4;
        const hipError_t e = launch_stream_pf<AK, EPI, 1, kStreamNTW>(kp, (int)al.list_len[4], s);
        if (e != hipSuccess || part == kPartShort) return e;
      }
      kp.list_idx = 5;
      return launch_wide<AK, EPI, kUp32 ? 32 : NVFP4_TALL_WN>(kp, (int)al.list_len[5], s);
    }
  }
  if (part == kPartTall) return hipSuccess;
  kp.list_idx = li;
  const int len = (int)al.list_len[li];
  switch (li) {
    case 0: return launch_stream_pf<AK, EPI, 1, kStreamNTW>(kp, len, s);
    case 1: return launch_stream_pf<AK, EPI, 2, kStreamNTW>(kp, len, s);
    case 2: return launch_lds<AK, EPI, 64, NVFP4_BIG_WN>(kp, len, s);
    default: return launch_lds<AK, EPI, 128, NVFP4_BIG_WN>(kp, len, s);
  }
}

KParams base_params(const GemmArgs& a) {
  KParams k{};
  k.T = a.T;
  k.topk = a.topk;
  k.I = a.I;
  k.plan = a.plan;
  k.g_w = a.g_w;
  return k;
}

}  // namespace

// Tile height from the mean rows per expert (host side, from dims only).
int pick_list(int64_t P, int slots) {
  const int64_t avg = P / (slots > 0 ? slots : 1);
  if (avg <= 16) return 0;
  if (avg <= 40) return 1;
  if (avg <= 96) return 2;
  return 3;
}

bool split_experts(const AlignShape& al) {
  return pick_list(al.P, al.slots) <= 1 && (al.T > 64 || (al.shared && al.T > kSplitRows));
}

bool prefers_decoded(int T, int topk, int E, int shared) {
  const AlignShape al = align_shape(T, topk, E, shared);
  return min(pick_list(al.P, al.slots), 3) >= NVFP4_WIDE_MIN_LIST || split_experts(al);
}

hipError_t launch_gemm1(const GemmArgs& a, bool w4a4, hipStream_t s) {
  const AlignShape al = align_shape(a.T, a.topk, a.E, a.shared);
  KParams k = base_params(a);
  k.N = 2 * a.I;
  k.K = a.H;
  k.sorted_pair = a.sorted_pair;
  k.a_rows = a.T;
  k.w_q = a.w_prep;
  k.w_sf = a.w_prep + (size_t)al.slots * k.N * (k.K / 2);
  if (w4a4) {
    k.a_q = a.a_q;
    k.a_sf = a.a_sf;
    k.a_h = a.a_h;
    k.g_a = a.g_a;
    k.g2 = a.g2;
    k.out_q = a.out_q;
    k.out_sf = a.out_sf;
    k.out_h = a.out_h;
    if (a.a_h) return launch_gemm<kActF16, kEpiSwigluFp4>(k, al, s, a.part);
    return launch_gemm<kActCodes, kEpiSwigluFp4>(k, al, s, a.part);
  }
  k.a_h = a.a_h;
  k.out_h = a.out_h;
  return launch_gemm<kActBf16, kEpiSwigluBf16>(k, al, s, a.part);
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t s) {
  AlignShape al = align_shape((int)a.M, 1, 1, 0);
  KParams k{};
  k.T = (int)a.M;
  k.topk = 1;
  k.N = (int)a.N;
  k.K = (int)a.K;
  k.plan = a.plan;
  k.sorted_pair = nullptr;   // row m of the output is row m of x
  k.a_rows = a.M;
  k.w_q = a.w_prep;
  k.w_sf = a.w_prep + (size_t)a.N * (a.K / 2);
  k.g_w = a.g_w;
  k.g_a = a.g_a;
  k.a_q = a.a_q;
  k.a_sf = a.a_sf;
  k.a_h = a.a_h;
  const bool f32 = a.out_dtype != 0;
  if (f32) k.out_f32 = static_cast<float*>(a.out);
  else k.out_h = static_cast<uint16_t*>(a.out);
  // Few rows from codes (at most 16) or bf16 (at most 4): K split over the
  // 4 wavefronts of a workgroup per 32 columns (N is a multiple of 128).
  // Measured at N = 34816, K = 5120: M = 1 W4A4 33.0 -> 30.3 us, W4A16
  // 35.7 -> 31.8 us, M = 16 W4A4 41.0 -> 39.7 us; W4A16 at M = 16 is faster
  // on the streaming kernel (35.7 against 47.1 us: its bf16 rows are 4x the
  // bytes of codes).
  if (a.M >= 1 && ((a.w4a4 && !a.a_h && a.M <= 16) || (!a.w4a4 && a.M <= 4))) {
    const dim3 grid((unsigned)(a.N / 32));
    if (a.w4a4) {
      if (f32) linear_splitk_kernel<kActCodes, true, 4><<<grid, 4 * kWave, 0, s>>>(k);
      else linear_splitk_kernel<kActCodes, false, 4><<<grid, 4 * kWave, 0, s>>>(k);
    } else {
      if (f32) linear_splitk_kernel<kActBf16, true, 4><<<grid, 4 * kWave, 0, s>>>(k);
      else linear_splitk_kernel<kActBf16, false, 4><<<grid, 4 * kWave, 0, s>>>(k);
    }
    return hipGetLastError();
  }
  if (!a.w4a4)
    return f32 ? launch_gemm<kActBf16, kEpiStoreF32>(k, al, s, kPartAll)
               : launch_gemm<kActBf16, kEpiStoreBf16>(k, al, s, kPartAll);
  if (a.a_h)
    return f32 ? launch_gemm<kActF16, kEpiStoreF32>(k, al, s, kPartAll)
               : launch_gemm<kActF16, kEpiStoreBf16>(k, al, s, kPartAll);
  return f32 ? launch_gemm<kActCodes, kEpiStoreF32>(k, al, s, kPartAll)
             : launch_gemm<kActCodes, kEpiStoreBf16>(k, al, s, kPartAll);
}

hipError_t launch_combine(const float* d, const int32_t* inv_pos, const float* topk_w, int T, int topk,
                          int shared, int H, void* out, int out_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 cgrid(T, (H + 1023) / 1024);
  // Non-temporal reads once the workspace exceeds half the 256 MB Infinity
  // Cache (measured: Zipf-skewed prefill, 537 MB, 127 -> 93 us; even
  // prefill, 268 MB, 53 -> 51 us; the 512-expert layer's 46 MB, 9.8 ->
  // 11.7 us, so small workspaces keep ordinary loads).
  const bool nt = (int64_t)T * (topk + shared) * H * 4 > (int64_t(128) << 20);
  if (out_dtype == 0) {
    if (nt) combine_kernel<true, true><<<cgrid, 256, 0, s>>>(d, inv_pos, topk_w, T, topk, shared, H, out);
    else combine_kernel<true, false><<<cgrid, 256, 0, s>>>(d, inv_pos, topk_w, T, topk, shared, H, out);
  } else {
    if (nt) combine_kernel<false, true><<<cgrid, 256, 0, s>>>(d, inv_pos, topk_w, T, topk, shared, H, out);
    else combine_kernel<false, false><<<cgrid, 256, 0, s>>>(d, inv_pos, topk_w, T, topk, shared, H, out);
  }
  return hipGetLastError();
}

hipError_t launch_gemm2_combine(const GemmArgs& a, bool w4a4, hipStream_t s) {
  const AlignShape al = align_shape(a.T, a.topk, a.E, a.shared);
  KParams k = base_params(a);
  k.N = a.H;
  k.K = a.I;
  k.sorted_pair = nullptr;
  k.a_rows = a.P;
  k.w_q = a.w_prep;
  k.w_sf = a.w_prep + (size_t)al.slots * k.N * (k.K / 2);
  k.out_f32 = a.d_ws;
  hipError_t e = hipSuccess;
  if (a.part != kPartCombine) {
    if (w4a4) {
      k.a_q = a.a_q;
      k.a_sf = a.a_sf;
      k.a_h = a.a_h;
      k.g_a = a.g_a;
      e = a.a_h ? launch_gemm<kActF16, kEpiStoreF32>(k, al, s, a.part)
                : launch_gemm<kActCodes, kEpiStoreF32>(k, al, s, a.part);
    } else {
      k.a_h = a.a_h;
      e = launch_gemm<kActBf16, kEpiStoreF32>(k, al, s, a.part);
    }
  }
  // The combine needs every row of d: it follows the whole GEMM, or runs
  // alone once both lists are done.
  if (e != hipSuccess || (a.part != kPartAll && a.part != kPartCombine)) return e;
  return launch_combine(a.d_ws, a.inv_pos, a.topk_w, a.T, a.topk, a.shared, a.H, a.out, a.out_dtype, s);
}

}  // namespace nvfp4
