// Grouped NVFP4 expert GEMMs with fused SwiGLU + requantisation (GEMM1) and
// the down projection + top-k weighted combine (GEMM2), for gfx950.
//
// Contraction strategy: NVFP4 operands are dequantised exactly in registers
// (code * E4M3 block scale, at most six significant bits) and multiplied on
// the 16x16x32 f16 (W4A4) or bf16 (W4A16) matrix instructions with FP32
// accumulation; the FP32 global scales enter as one per-expert alpha in the
// epilogue (the alpha-pointer-array epilogue with beta = 0 of vLLM PR #29242,
// review of nvfp4_blockwise_moe_kernel.cu).  The native FP4 instructions of
// gfx950 take power-of-two scales per 32 elements, which cannot carry E4M3
// scales per 16 exactly; see the design doc for the comparison.
//
// Work decomposition: the alignment plan lists (expert, 16..128-row tile)
// pairs on the device; a workgroup takes one tile and BN = 4 * WN output
// columns.  Each wavefront owns WN columns for all BM rows: it streams its
// weight columns straight from HBM into registers (one coalesced 16-byte load
// per lane per 16 columns x 128 k, see prep.hip) while the BM x 128 activation
// chunk is staged once per workgroup in LDS, dequantised, double-buffered.
// Workgroup ids are remapped so that consecutive tiles land on the same XCD
// (shared L2 for the expert's weights and the tile's activation rows).
#include "common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

// Tile configuration (compile-time; the defaults are the measured best).
#ifndef NVFP4_DIRECT_NTW
#define NVFP4_DIRECT_NTW 2     // 16-column tiles per wavefront, short-tile kernel
#endif
#ifndef NVFP4_DIRECT_PFMAX
#define NVFP4_DIRECT_PFMAX 4   // deepest register prefetch ring (128-k chunks)
#endif
#ifndef NVFP4_LIST_MAX
#define NVFP4_LIST_MAX 2       // tallest tile list used (2: 64 rows, 3: 128 rows)
#endif
#ifndef NVFP4_BIG_WN
#define NVFP4_BIG_WN 32        // columns per wavefront, LDS-staged kernel
#endif
#ifndef NVFP4_BIG_NW
#define NVFP4_BIG_NW 4         // wavefronts per workgroup, LDS-staged kernel
#endif
#ifndef NVFP4_DIRECT_AF16
#define NVFP4_DIRECT_AF16 0    // short tiles: stage activations dequantised (f16)
#endif

constexpr int kNW = 4;      // wavefronts per workgroup
constexpr int kBK = 128;    // contraction chunk
constexpr int kLDA = kBK + 8;  // LDS row stride in 16-bit elements (272 bytes)

enum Epi { kEpiSwigluFp4 = 0, kEpiSwigluBf16 = 1, kEpiStoreF32 = 2 };

struct KParams {
  int T, topk, I, N, K;
  int n_blocks;
  int list_idx;            // which plan list (tile height)
  const int32_t* offsets;
  const int32_t* sorted_pair;  // GEMM1: row -> pair; GEMM2: null (row is the A row)
  const int32_t* plan;
  const uint8_t* a_q;
  const uint8_t* a_sf;
  const uint16_t* a_bf16;
  const float* g_a;
  const uint8_t* w_q;      // prepped codes
  const uint8_t* w_sf;     // prepped scales
  const float* g_w;
  const float* g2;
  uint8_t* out_q;
  uint8_t* out_sf;
  uint16_t* out_bf16;
  float* out_f32;
};

// Bijection from the launch order to the work order such that each XCD (the
// hardware deals workgroups round-robin over 8 XCDs) receives a contiguous
// range of work items.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int q = G >> 3, r = G & 7, x = bid & 7, idx = bid >> 3;
  return x * q + min(x, r) + idx;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Epilogue of a wavefront's MT x NTW accumulator tiles (rows row0 + [0, 16 MT),
// columns n_wave0 + [0, 16 NTW) of the streaming column order).
template <int EPI, int MT, int NTW>
__device__ __forceinline__ void epilogue(const KParams& p, f32x4 (&acc)[MT][NTW], int e, int row0,
                                         int nrows, int n_wave0, int lane) {
  const float alpha = p.g_a ? (*p.g_a) * p.g_w[e] : p.g_w[e];
  const int ln = lane & 15, lg = lane >> 4;
  if constexpr (EPI == kEpiStoreF32) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + lg * 4 + r;
          if (row < nrows)
            p.out_f32[(int64_t)(row0 + row) * p.N + n_wave0 + 16 * j + ln] = alpha * acc[i][j][r];
        }
  } else {
    const float g2 = (EPI == kEpiSwigluFp4) ? *p.g2 : 0.0f;
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
          h[r] = silu(gate) * up;
        }
        if constexpr (EPI == kEpiSwigluFp4) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float am = row16_max(fabsf(h[r]));
            const uint32_t sc = e4m3_scale_code(am, g2);
            const E2M1Bounds bd = e2m1_bounds(e4m3_value(sc), g2);
            const uint32_t code = e2m1_code(h[r], bd, sc == 0);
            const uint32_t other = (uint32_t)dpp_xor1_i((int)code);
            const int row = i * 16 + lg * 4 + r;
            if (row < nrows) {
              const int64_t pr = row0 + row;
              if ((ln & 1) == 0)
                p.out_q[pr * (p.I >> 1) + hb * 8 + (ln >> 1)] = (uint8_t)(code | (other << 4));
              if (ln == 0) p.out_sf[pr * (p.I >> 4) + hb] = (uint8_t)sc;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = i * 16 + lg * 4 + r;
            if (row < nrows)
              p.out_bf16[(int64_t)(row0 + row) * p.I + hb * 16 + ln] = (uint16_t)f32_to_bf16_bits(h[r]);
          }
        }
      }
  }
}

// Work item of this workgroup: (expert, first row, valid rows, column block).
struct Tile {
  int e, row0, nrows, nb;
};
// Tiles whose work shares data are kept on one XCD (``remap``): the launch
// order is mapped so that each XCD receives a contiguous range of tiles.
__device__ __forceinline__ bool decode_tile(const KParams& p, bool remap, Tile& t) {
  const int ntiles = p.plan[p.list_idx];
  const int G = ntiles * p.n_blocks;
  if ((int)blockIdx.x >= G) return false;
  const int v = remap ? xcd_remap(blockIdx.x, G) : (int)blockIdx.x;
  const int tile = v / p.n_blocks;
  t.nb = v - tile * p.n_blocks;
  const int* ent = p.plan + p.plan[4 + p.list_idx] + 2 * tile;
  t.e = ent[0] & 2047;
  const uint32_t rr = (uint32_t)ent[1];
  t.row0 = (int)(rr & 0xFFFFFFu);
  t.nrows = (int)(rr >> 24);
  return true;
}

template <bool W4A4, int EPI, int BM, int WN, int NW>
__global__ __launch_bounds__(NW * kWave) void grouped_gemm_kernel(KParams p) {
  constexpr int MT = BM / 16;
  constexpr int NTW = WN / 16;
  static_assert(NTW % 2 == 0, "scale words cover column tiles in pairs");
  // A staging pieces per chunk: 16-byte pieces of codes (32 elements) for
  // W4A4, 16-byte pieces of bf16 (8 elements) for W4A16.
  constexpr int PIECES = W4A4 ? BM * 4 : BM * 16;
  static_assert(PIECES % (NW * kWave) == 0, "staging pieces split evenly over the threads");
  constexpr int PPT = PIECES / (NW * kWave);
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLDA];

  Tile t;
  if (!decode_tile(p, true, t)) return;
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
    const int r = W4A4 ? (pc >> 2) : (pc >> 4);
    const int qq = W4A4 ? (pc & 3) : (pc & 15);
    int src = t.row0 + min(r, t.nrows - 1);
    if (p.sorted_pair) src = pair_token(p.sorted_pair[src], p.T, p.topk);
    if constexpr (W4A4) {
      a_src[j] = p.a_q + (int64_t)src * (K >> 1) + qq * 16;
      s_src[j] = p.a_sf + (int64_t)src * (K >> 4) + qq * 2;
      a_dst[j] = r * kLDA + qq * 32;
    } else {
      a_src[j] = reinterpret_cast<const uint8_t*>(p.a_bf16 + (int64_t)src * K + qq * 8);
      s_src[j] = nullptr;
      a_dst[j] = r * kLDA + qq * 8;
    }
  }
  u32x4 a_reg[PPT];
  uint32_t a_sreg[PPT];
  auto load_a = [&](int kc) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      if constexpr (W4A4) {
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
      if constexpr (W4A4) {
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
  const int64_t sbase = ((int64_t)(t.e * (NT >> 1) + (nt0 >> 1)) * KC) * kWave + lane;
  u32x4 bq0[NTW], bq1[NTW];
  uint32_t bs0[NTW / 2], bs1[NTW / 2];
  auto load_b = [&](int kc, u32x4 (&bq)[NTW], uint32_t (&bs)[NTW / 2]) {
    if (!wave_on) return;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
      bq[j] = *reinterpret_cast<const u32x4*>(p.w_q + (wbase + ((int64_t)j * KC + kc) * kWave) * 16);
#pragma unroll
    for (int j = 0; j < NTW / 2; ++j)
      bs[j] = *reinterpret_cast<const uint32_t*>(p.w_sf + (sbase + ((int64_t)j * KC + kc) * kWave) * 4);
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
    if constexpr (W4A4) {
      f16x2 sb2[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) sb2[j] = e4m3x2_to_f16x2(bs[j >> 1] >> ((j & 1) * 16));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          bf[j] = dequant8_f16(bq[j][s], s < 2 ? f16x2_lo(sb2[j]) : f16x2_hi(sb2[j]));
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
        const uint32_t w = bs[j >> 1] >> ((j & 1) * 16);
        sb[j][0] = e4m3_value(w & 0xFFu);
        sb[j][1] = e4m3_value((w >> 8) & 0xFFu);
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
  for (int kc = 0;; kc += 2) {
    const bool more1 = kc + 1 < KC;
    if (more1) {
      load_a(kc + 1);
      load_b(kc + 1, bq1, bs1);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(0, bq0, bs0);
    __builtin_amdgcn_sched_barrier(0);
    if (!more1) break;
    store_a(1);
    __syncthreads();
    const bool more2 = kc + 2 < KC;
    if (more2) {
      load_a(kc + 2);
      load_b(kc + 2, bq0, bs0);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(1, bq1, bs1);
    __builtin_amdgcn_sched_barrier(0);
    if (!more2) break;
    store_a(0);
    __syncthreads();
  }
  if (!wave_on) return;
  epilogue<EPI, MT, NTW>(p, acc, t.e, t.row0, t.nrows, n_wave0, lane);
}

// Main loop for short tiles (16 or 32 rows), the decode regime where the
// weights are read once and the path is bound by HBM bandwidth.  The tile's
// activation rows (packed NVFP4 or bf16, all of K) are staged into LDS once,
// behind a single barrier; after that every wavefront only streams its own
// weight columns, through a register ring of PF 128-k chunks, so PF chunks of
// loads are in flight while the matrix instructions consume the oldest one.
// Activation fragments use the weights' lane layout: lane 16g + m reads the
// 32 k values [32g, 32g + 32) of row m of a chunk.
template <bool W4A4, int EPI, int MT, int NTW, int PF>
__global__ __launch_bounds__(kNW * kWave) void grouped_gemm_direct_kernel(KParams p) {
  constexpr int BM = MT * 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];
  Tile t;
  // Column blocks of a tile read disjoint weights: no XCD grouping needed.
  if (!decode_tile(p, false, t)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_wave0 = (t.nb * kNW + wv) * (NTW * 16);
  const bool wave_on = n_wave0 < p.N;
  const int K = p.K, KC = K / kBK, NT = p.N / 16;
  const int g = lane >> 4;

  const int nt0 = n_wave0 >> 4;
  const int64_t wbase = ((int64_t)(t.e * NT + nt0) * KC) * kWave + lane;
  const int64_t sbase = ((int64_t)(t.e * (NT >> 1) + (nt0 >> 1)) * KC) * kWave + lane;
  u32x4 bq[PF][NTW];
  uint32_t bs[PF][NTW / 2];
  // bf16 activation fragments ride in the ring too (W4A16: a bf16 tile is 4x
  // the packed size, too large to stage whole in LDS without costing
  // occupancy).  Rows past the tile end read a valid row; never stored.
  constexpr int AR = W4A4 ? 1 : MT;
  u32x4 ab[PF][AR][W4A4 ? 1 : 4];
  int64_t arow_g[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    int src = t.row0 + min(i * 16 + (lane & 15), t.nrows - 1);
    if (!W4A4 && p.sorted_pair) src = pair_token(p.sorted_pair[src], p.T, p.topk);
    arow_g[i] = src;
  }
  auto load = [&](int kc, int u) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int64_t unit = wbase + ((int64_t)j * KC + kc) * kWave;
      bq[u][j] = *reinterpret_cast<const u32x4*>(p.w_q + unit * 16);
    }
#pragma unroll
    for (int j = 0; j < NTW / 2; ++j) {
      const int64_t unit = sbase + ((int64_t)j * KC + kc) * kWave;
      bs[u][j] = *reinterpret_cast<const uint32_t*>(p.w_sf + unit * 4);
    }
    if constexpr (!W4A4) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          ab[u][i][s4] = *reinterpret_cast<const u32x4*>(p.a_bf16 + arow_g[i] * K + kc * kBK + g * 32 + s4 * 8);
    }
  };
  // The weight stream does not depend on the activations: start it first,
  // in slot order (the compiler would otherwise cluster the loads by type,
  // and every later wait would have to drain the ring).
  if (wave_on) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- W4A4: stage the tile's activation rows (rows past the tile end
  // repeat the last valid row; their results are never stored), packed, or
  // dequantised to f16 once for all wavefronts (AF16).  Row stride is padded
  // by 16 bytes so the 16 rows read by one fragment load spread over the
  // banks.
  constexpr bool AF16 = W4A4 && NVFP4_DIRECT_AF16;
  const int row_bytes = K >> 1;
  const int stride = AF16 ? K * 2 + 16 : row_bytes + 16;
  const int sf_bytes = K >> 4;
  uint8_t* a_sf_lds = a_lds + BM * stride;
  if constexpr (AF16) {
    const int pieces = K >> 5;  // 32-element pieces per row
    for (int pc = tid; pc < BM * pieces; pc += kNW * kWave) {
      const int r = pc / pieces, c = pc - r * pieces;
      int src = t.row0 + min(r, t.nrows - 1);
      if (p.sorted_pair) src = pair_token(p.sorted_pair[src], p.T, p.topk);
      const u32x4 cw = *reinterpret_cast<const u32x4*>(p.a_q + (int64_t)src * row_bytes + c * 16);
      const f16x2 s2 = e4m3x2_to_f16x2(
          *reinterpret_cast<const uint16_t*>(p.a_sf + (int64_t)src * sf_bytes + c * 2));
      uint8_t* dst = a_lds + r * stride + c * 64;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        *reinterpret_cast<f16x8*>(dst + 16 * w) = dequant8_f16(cw[w], w < 2 ? f16x2_lo(s2) : f16x2_hi(s2));
    }
    __syncthreads();
  } else if constexpr (W4A4) {
    const int pieces = row_bytes >> 4;  // 16-byte pieces per row
    for (int pc = tid; pc < BM * pieces; pc += kNW * kWave) {
      const int r = pc / pieces, c = pc - r * pieces;
      int src = t.row0 + min(r, t.nrows - 1);
      if (p.sorted_pair) src = pair_token(p.sorted_pair[src], p.T, p.topk);
      *reinterpret_cast<u32x4*>(a_lds + r * stride + c * 16) =
          *reinterpret_cast<const u32x4*>(p.a_q + (int64_t)src * row_bytes + c * 16);
    }
    const int spieces = sf_bytes >> 1;  // 2-byte pieces per row
    for (int pc = tid; pc < BM * spieces; pc += kNW * kWave) {
      const int r = pc / spieces, c = pc - r * spieces;
      int src = t.row0 + min(r, t.nrows - 1);
      if (p.sorted_pair) src = pair_token(p.sorted_pair[src], p.T, p.topk);
      *reinterpret_cast<uint16_t*>(a_sf_lds + r * sf_bytes + c * 2) =
          *reinterpret_cast<const uint16_t*>(p.a_sf + (int64_t)src * sf_bytes + c * 2);
    }
    __syncthreads();
  }
  if (!wave_on) return;  // no barriers below

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = lane & 15;
  auto compute = [&](int kc, int u) {
    // Packed activation fragments of this chunk for every m-tile (W4A4), and
    // the f16 block scales of this chunk ({k-steps 0-1, k-steps 2-3}).
    u32x4 aq[MT];
    f16x2 sa2[MT], sb2[NTW];
    if constexpr (W4A4) {
#pragma unroll
      for (int i = 0; i < MT && !AF16; ++i) {
        aq[i] = *reinterpret_cast<const u32x4*>(a_lds + (i * 16 + arow) * stride + kc * 64 + g * 16);
        sa2[i] = e4m3x2_to_f16x2(*reinterpret_cast<const uint16_t*>(
            a_sf_lds + (i * 16 + arow) * sf_bytes + kc * 8 + g * 2));
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j) sb2[j] = e4m3x2_to_f16x2(bs[u][j >> 1] >> ((j & 1) * 16));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int sh = (s < 2 ? 0 : 8);
      if constexpr (W4A4) {
        f16x8 bf[NTW], af[MT];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          bf[j] = dequant8_f16(bq[u][j][s], s < 2 ? f16x2_lo(sb2[j]) : f16x2_hi(sb2[j]));
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if constexpr (AF16)
            af[i] = *reinterpret_cast<const f16x8*>(a_lds + (i * 16 + arow) * stride +
                                                     (kc * kBK + g * 32 + s * 8) * 2);
          else
            af[i] = dequant8_f16(aq[i][s], s < 2 ? f16x2_lo(sa2[i]) : f16x2_hi(sa2[i]));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      } else {
        bf16x8 bf[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const uint32_t sb = (bs[u][j >> 1] >> ((j & 1) * 16 + sh)) & 0xFFu;
          bf[j] = dequant8_bf16(bq[u][j][s], e4m3_value(sb));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, ab[u][i][s]);
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // PF divides KC (chosen by the launcher): the prologue above, a steady
  // state with unconditional loads, then the drain.  The scheduling fences
  // pin each refill right behind the compute that frees its slot (left
  // alone, the scheduler sinks all refills to the end of the loop body and
  // the ring runs empty).
  for (int kc0 = PF; kc0 < KC; kc0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      compute(kc0 - PF + u, u);
      __builtin_amdgcn_sched_barrier(0);
      load(kc0 + u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < PF; ++u) compute(KC - PF + u, u);
  epilogue<EPI, MT, NTW>(p, acc, t.e, t.row0, t.nrows, n_wave0, lane);
}

// Largest activation tile the short-tile kernel stages (larger ones, e.g. bf16
// rows with a long K, take the chunked LDS kernel instead).
constexpr size_t kDirectLdsMax = 96 * 1024;

// LDS bytes of the short-tile kernel: padded packed activation rows + scales
// (W4A4 only; the bf16 variant keeps its activations in registers).
size_t direct_lds_bytes(bool w4a4, int BM, int K) {
  if (!w4a4) return 0;
  if (NVFP4_DIRECT_AF16) return (size_t)BM * (K * 2 + 16) + (size_t)BM * (K / 16);
  return (size_t)BM * (K / 2 + 16) + (size_t)BM * (K / 16);
}

// out[t] = sum_j w[t][j] * d[inv_pos[t*k + j]] (+ shared row), FP32, j ascending.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ d,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int topk, int shared, int H, void* out) {
  const int t = blockIdx.x;
  {
    const int c = blockIdx.y * 1024 + threadIdx.x * 4;
    if (c >= H) return;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
      const int pos = inv_pos[(int64_t)t * topk + j];
      if (pos >= 0) {
        const float w = topk_w[(int64_t)t * topk + j];
        const f32x4 x = *reinterpret_cast<const f32x4*>(d + (int64_t)pos * H + c);
        a += w * x;
      }
    }
    if (shared) {
      const int pos = inv_pos[(int64_t)T * topk + t];
      if (pos >= 0) a += *reinterpret_cast<const f32x4*>(d + (int64_t)pos * H + c);
    }
    if constexpr (BF16) {
      uint32_t lo = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
      uint32_t hi = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + (int64_t)t * H + c) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)t * H + c) = a;
    }
  }
}

// Tile height from the mean rows per expert (host side, from dims only).
int pick_list(int64_t P, int slots) {
  const int64_t avg = P / (slots > 0 ? slots : 1);
  if (avg <= 16) return 0;
  if (avg <= 40) return 1;
  if (avg <= 96) return 2;
  return 3;
}

template <bool W4A4, int EPI, int BM, int WN>
hipError_t launch_one(KParams kp, int list_len, hipStream_t s) {
  constexpr int NW = NVFP4_BIG_NW;
  kp.n_blocks = (kp.N + NW * WN - 1) / (NW * WN);
  const int64_t G = (int64_t)list_len * kp.n_blocks;
  const int64_t grid = (G + 7) / 8 * 8;
  grouped_gemm_kernel<W4A4, EPI, BM, WN, NW><<<(unsigned)grid, NW * kWave, 0, s>>>(kp);
  return hipGetLastError();
}

template <bool W4A4, int EPI, int MT, int NTW, int PF>
hipError_t launch_direct(const KParams& kp, int list_len, hipStream_t s) {
  const int64_t G = (int64_t)list_len * kp.n_blocks;
  const int64_t grid = (G + 7) / 8 * 8;
  const size_t lds = direct_lds_bytes(W4A4, MT * 16, kp.K);
  auto kern = grouped_gemm_direct_kernel<W4A4, EPI, MT, NTW, PF>;
  static bool attr_set = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kDirectLdsMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<(unsigned)grid, kNW * kWave, lds, s>>>(kp);
  return hipGetLastError();
}

// Prefetch depth: the largest of 8, 6, 4, 3, 2, 1 chunks that divides the
// chunk count (fewer for bf16 activations, whose fragments are 4x larger).
template <bool W4A4, int EPI, int MT, int NTW>
hipError_t launch_direct_pf(const KParams& kp, int len, hipStream_t s) {
  const int KC = kp.K / kBK;
  if (NVFP4_DIRECT_PFMAX >= 8 && W4A4 && KC % 8 == 0)
    return launch_direct<W4A4, EPI, MT, NTW, 8>(kp, len, s);
  if (NVFP4_DIRECT_PFMAX >= 6 && W4A4 && KC % 6 == 0)
    return launch_direct<W4A4, EPI, MT, NTW, 6>(kp, len, s);
  if (KC % 4 == 0) return launch_direct<W4A4, EPI, MT, NTW, 4>(kp, len, s);
  if (KC % 3 == 0) return launch_direct<W4A4, EPI, MT, NTW, 3>(kp, len, s);
  if (KC % 2 == 0) return launch_direct<W4A4, EPI, MT, NTW, 2>(kp, len, s);
  return launch_direct<W4A4, EPI, MT, NTW, 1>(kp, len, s);
}

template <bool W4A4, int EPI>
hipError_t launch_gemm(KParams kp, const AlignShape& al, hipStream_t s) {
  const int li = min(pick_list(al.P, al.slots), NVFP4_LIST_MAX);
  kp.list_idx = li;
  const int wn = li <= 1 ? 16 * NVFP4_DIRECT_NTW : 64;
  kp.n_blocks = (kp.N + kNW * wn - 1) / (kNW * wn);
  const int len = (int)al.list_len[li];
  if (li <= 1 && direct_lds_bytes(W4A4, li == 0 ? 16 : 32, kp.K) > kDirectLdsMax) {
    kp.list_idx = 2;
    return launch_one<W4A4, EPI, 64, NVFP4_BIG_WN>(kp, (int)al.list_len[2], s);
  }
  switch (li) {
    case 0: return launch_direct_pf<W4A4, EPI, 1, NVFP4_DIRECT_NTW>(kp, len, s);
    case 1: return launch_direct_pf<W4A4, EPI, 2, NVFP4_DIRECT_NTW>(kp, len, s);
    case 2: return launch_one<W4A4, EPI, 64, NVFP4_BIG_WN>(kp, len, s);
    default: return launch_one<W4A4, EPI, 128, NVFP4_BIG_WN>(kp, len, s);
  }
}

KParams base_params(const GemmArgs& a) {
  KParams k{};
  k.T = a.T;
  k.topk = a.topk;
  k.I = a.I;
  k.offsets = a.offsets;
  k.plan = a.plan;
  k.g_w = a.g_w;
  return k;
}

}  // namespace

hipError_t launch_gemm1(const GemmArgs& a, bool w4a4, hipStream_t s) {
  const AlignShape al = align_shape(a.T, a.topk, a.E, a.shared);
  KParams k = base_params(a);
  k.N = 2 * a.I;
  k.K = a.H;
  k.sorted_pair = a.sorted_pair;
  k.w_q = a.w_prep;
  k.w_sf = a.w_prep + (size_t)al.slots * k.N * (k.K / 2);
  if (w4a4) {
    k.a_q = a.a_q;
    k.a_sf = a.a_sf;
    k.g_a = a.g_a;
    k.g2 = a.g2;
    k.out_q = a.out_q;
    k.out_sf = a.out_sf;
    return launch_gemm<true, kEpiSwigluFp4>(k, al, s);
  }
  k.a_bf16 = a.a_bf16;
  k.out_bf16 = a.out_bf16;
  return launch_gemm<false, kEpiSwigluBf16>(k, al, s);
}

hipError_t launch_gemm2_combine(const GemmArgs& a, bool w4a4, hipStream_t s) {
  const AlignShape al = align_shape(a.T, a.topk, a.E, a.shared);
  KParams k = base_params(a);
  k.N = a.H;
  k.K = a.I;
  k.sorted_pair = nullptr;
  k.w_q = a.w_prep;
  k.w_sf = a.w_prep + (size_t)al.slots * k.N * (k.K / 2);
  k.out_f32 = a.d_ws;
  hipError_t e;
  if (w4a4) {
    k.a_q = a.a_q;
    k.a_sf = a.a_sf;
    k.g_a = a.g_a;
    e = launch_gemm<true, kEpiStoreF32>(k, al, s);
  } else {
    k.a_bf16 = a.a_bf16;
    e = launch_gemm<false, kEpiStoreF32>(k, al, s);
  }
  if (e != hipSuccess) return e;
  if (a.T == 0) return hipSuccess;
  const dim3 cgrid(a.T, (a.H + 1023) / 1024);
  if (a.out_dtype == 0)
    combine_kernel<true><<<cgrid, 256, 0, s>>>(a.d_ws, a.inv_pos, a.topk_w, a.T, a.topk, a.shared, a.H, a.out);
  else
    combine_kernel<false><<<cgrid, 256, 0, s>>>(a.d_ws, a.inv_pos, a.topk_w, a.T, a.topk, a.shared, a.H, a.out);
  return hipGetLastError();
}

}  // namespace nvfp4
