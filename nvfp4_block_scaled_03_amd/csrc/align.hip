// Router and permutation by expert (gfx950).
//
// moe_align groups the (token, expert) pairs by expert with a stable order --
// the grouped-GEMM metadata step (get_cutlass_moe_mm_data) of vLLM PR #29242
// -- without atomics deciding any position: per-chunk histograms, a per-expert
// scan, then a scatter whose in-chunk ranks come from wavefront ballots.  It
// also writes the tile lists the grouped GEMMs read, so per-expert problem
// sizes never leave the device (vLLM PR #29242, debug trace: the host problem
// shape is not available to the grouped GEMM).
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "quant.h"

namespace nvfp4 {
namespace {

struct AlignP {
  const int32_t* ids;
  int T, topk, E, shared, slots, nchunks;
  int64_t P;
};

__device__ __forceinline__ int expert_of(const AlignP& a, int64_t f, bool& valid) {
  const int64_t tk = (int64_t)a.T * a.topk;
  if (f < tk) {
    const int e = a.ids ? a.ids[f] : 0;   // no ids: every pair to expert 0 (dense use)
    valid = e >= 0 && e < a.E;
    return e;
  }
  valid = true;
  return a.E;  // shared expert slot
}

// ---------------------------------------------------------------- counts
// Expert histogram of one chunk of kAlignChunk pairs (256 threads).
__device__ __forceinline__ void count_chunk(const AlignP& a, int32_t* __restrict__ counts, int chunk) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < a.slots; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)chunk * kAlignChunk;
  for (int r = 0; r < kAlignChunk / 256; ++r) {
    const int64_t f = f0 + r * 256 + threadIdx.x;
    if (f < a.P) {
      bool valid;
      const int e = expert_of(a, f, valid);
      if (valid) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.slots; e += 256)
    counts[(int64_t)chunk * a.slots + e] = hist[e];
}

__global__ __launch_bounds__(256) void align_count_kernel(AlignP a, int32_t* __restrict__ counts) {
  count_chunk(a, counts, blockIdx.x);
}

// Exclusive scan over 1024 threads; returns the thread's prefix, *total gets the sum.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int s = wsum[i];
    base += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// One tile-list entry: {expert | m_tile << 11, first row | rows << 24}, so a
// GEMM workgroup learns its expert, rows and row count from one 8-byte read.
// Expert e owns rows [start, start + n).
__device__ __forceinline__ void write_tile(int32_t* dst, int e, int mt, int BM, int start, int n) {
  const int row0 = start + mt * BM;
  const int rows = min(BM, n - mt * BM);
  dst[0] = e | (mt << 11);
  dst[1] = (int32_t)((uint32_t)row0 | ((uint32_t)rows << 24));
}

// Tiles [0, nt) of expert e (rows [start, start + n), height BM) at
// plan[pos + 2 mt].  A lane whose expert has at most kOwnTiles tiles writes
// them itself; the tiles of a larger expert (skewed routing gives one expert
// thousands of rows, hundreds of tiles per list) are written by all 64 lanes
// of its wavefront, one such expert at a time, instead of by one lane in
// series.  Every lane of the wavefront must call this (wave-wide ballot).
// A threshold that even routing reaches would serialise whole wavefronts,
// so it sits above the tiles of an evenly shared P <= 4096.
constexpr int kOwnTiles = 32;
__device__ __forceinline__ void write_tiles(int32_t* __restrict__ plan, int pos, int nt, int e, int BM,
                                            int start, int n) {
  const bool own = nt <= kOwnTiles;
  if (own)
    for (int mt = 0; mt < nt; ++mt) write_tile(plan + pos + 2 * mt, e, mt, BM, start, n);
  uint64_t heavy = __ballot(!own);
  const int lane = threadIdx.x & 63;
  while (heavy) {
    const int src = __builtin_ctzll(heavy);
    heavy &= heavy - 1;
    const int pos_s = __builtin_amdgcn_readlane(pos, src), nt_s = __builtin_amdgcn_readlane(nt, src);
    const int e_s = __builtin_amdgcn_readlane(e, src), start_s = __builtin_amdgcn_readlane(start, src);
    const int n_s = __builtin_amdgcn_readlane(n, src);
    for (int mt = lane; mt < nt_s; mt += 64) write_tile(plan + pos_s + 2 * mt, e_s, mt, BM, start_s, n_s);
  }
}

// Exclusive scan of V values per thread over 1024 threads (one pass, two
// barriers); tot[v] receives the sums.
template <int V>
__device__ void block_exclusive_scan_1024_v(const int (&v)[V], int (&out)[V], int (&tot)[V]) {
  __shared__ int wsum[16][V];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x[V];
#pragma unroll
  for (int i = 0; i < V; ++i) x[i] = v[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int y = __shfl_up(x[i], off);
      if (lane >= off) x[i] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < V; ++i) wsum[w][i] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int base = 0, t = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int s = wsum[j][i];
      base += j < w ? s : 0;
      t += s;
    }
    out[i] = base + x[i] - v[i];
    tot[i] = t;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- plan (one workgroup)
// The tile lists in the one-workgroup alignment (P <= kSmallP), where one
// scan of four values serves the expert offsets and all six lists: the
// per-expert tile counts travel two per int (16 bits each: a list holds at
// most P / 16 + slots <= 1280 tiles, so no half-sum carries into the other
// half).  plan_counts_small packs the counts; write_plan_small writes the
// header and the expert's tiles from the scan of the packed counts.
__device__ __forceinline__ void plan_counts_small(int e, int slots, int n_e, int (&packed)[3]) {
  int tiles[kPlanLists];
#pragma unroll
  for (int b = 0; b < kPlanLists; ++b)
    tiles[b] = (e < slots && plan_list_has(b, n_e)) ? (n_e + kPlanBMs[b] - 1) / kPlanBMs[b] : 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) packed[i] = tiles[2 * i] | (tiles[2 * i + 1] << 16);
}

__device__ __forceinline__ void write_plan_small(int32_t* __restrict__ plan, const PlanOffs& lo, int e,
                                                 int slots, int off_e, int n_e, const int (&pstart)[3],
                                                 const int (&ptot)[3]) {
  static_assert(kPlanLists == 6, "three ints of two 16-bit counts");
  if (e == 0) {
#pragma unroll
    for (int b = 0; b < kPlanLists; ++b) {
      plan[b] = (ptot[b >> 1] >> (16 * (b & 1))) & 0xFFFF;
      plan[kPlanLists + b] = lo.v[b];
    }
  }
#pragma unroll
  for (int b = 0; b < kPlanLists; ++b) {
    const int t0 = (pstart[b >> 1] >> (16 * (b & 1))) & 0xFFFF;
    const int nt = (e < slots && plan_list_has(b, n_e)) ? (n_e + kPlanBMs[b] - 1) / kPlanBMs[b] : 0;
    write_tiles(plan, lo.v[b] + 2 * t0, nt, e, kPlanBMs[b], off_e, n_e);
  }
}

// Per expert: turn the per-chunk counts into the chunk's first output row
// (in place), then scan over experts and write the offsets.
// Up to kScanRegChunks chunks (P <= 65536) every count is loaded at once and
// the per-expert prefixes stay in registers until the expert offset is
// known: one memory latency in all.  Beyond that both walks over the chunks
// load a group of chunks together (independent loads), so each costs one
// memory latency per group.
constexpr int kScanGroup = 16;
constexpr int kScanRegChunks = 64;
__device__ __forceinline__ void scan_body(const AlignP& a, int32_t* __restrict__ counts,
                                          int32_t* __restrict__ offsets) {
  const int e = threadIdx.x;
  const bool in_regs = a.nchunks <= kScanRegChunks;
  int n_e = 0;
  int pre[kScanRegChunks];
  if (e < a.slots && in_regs) {
#pragma unroll
    for (int j = 0; j < kScanRegChunks; ++j) pre[j] = j < a.nchunks ? counts[(int64_t)j * a.slots + e] : 0;
#pragma unroll
    for (int j = 0; j < kScanRegChunks; ++j) {
      const int v = pre[j];
      pre[j] = n_e;  // exclusive prefix
      n_e += v;
    }
  } else if (e < a.slots) {
    for (int c0 = 0; c0 < a.nchunks; c0 += kScanGroup) {
      int v[kScanGroup];
#pragma unroll
      for (int j = 0; j < kScanGroup; ++j)
        v[j] = c0 + j < a.nchunks ? counts[(int64_t)(c0 + j) * a.slots + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanGroup; ++j) {
        if (c0 + j < a.nchunks) counts[(int64_t)(c0 + j) * a.slots + e] = n_e;  // exclusive prefix
        n_e += v[j];
      }
    }
  }
  int total;
  const int off_e = block_exclusive_scan_1024(n_e, &total);
  if (e < a.slots && in_regs) {
#pragma unroll
    for (int j = 0; j < kScanRegChunks; ++j)
      if (j < a.nchunks) counts[(int64_t)j * a.slots + e] = pre[j] + off_e;
    offsets[e] = off_e;
  } else if (e < a.slots) {
    for (int c0 = 0; c0 < a.nchunks; c0 += kScanGroup) {
      int v[kScanGroup];
#pragma unroll
      for (int j = 0; j < kScanGroup; ++j)
        v[j] = c0 + j < a.nchunks ? counts[(int64_t)(c0 + j) * a.slots + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanGroup; ++j)
        if (c0 + j < a.nchunks) counts[(int64_t)(c0 + j) * a.slots + e] = v[j] + off_e;
    }
    offsets[e] = off_e;
  }
  if (e == 0) offsets[a.slots] = total;
}

// (the tile lists are written by the scatter launch)
__global__ __launch_bounds__(1024) void align_scan_kernel(AlignP a, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets) {
  scan_body(a, counts, offsets);
}

// ---------------------------------------------------------------- scatter
// Places the pairs of one chunk: each pair's row is its expert's base for
// the chunk plus its rank among the chunk's earlier pairs of that expert
// (wavefront ballots within a round of 256, LDS counts across wavefronts and
// rounds), so the order is stable and no atomic decides a position.
// lds: 5 kMaxExperts ints.
constexpr int kScatterLds = 5 * kMaxExperts;
__device__ __forceinline__ void scatter_chunk(const AlignP& a, const int32_t* __restrict__ bases,
                                              int32_t* __restrict__ sorted_pair,
                                              int32_t* __restrict__ inv_pos, int chunk, int* lds) {
  int* const running = lds;
  int (*const wcnt)[kMaxExperts] = reinterpret_cast<int (*)[kMaxExperts]>(lds + kMaxExperts);
  for (int e = threadIdx.x; e < a.slots; e += 256) {
    running[e] = bases[(int64_t)chunk * a.slots + e];
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kAlignChunk / 256; ++r) {
    const int64_t f = (int64_t)chunk * kAlignChunk + r * 256 + threadIdx.x;
    const bool in = f < a.P;
    bool valid = false;
    int e = in ? expert_of(a, f, valid) : 0;
    valid = valid && in;
    const int key = valid ? e : 2047;
    uint64_t same = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) {
      const bool b = (key >> bit) & 1;
      const uint64_t bal = __ballot(b);
      same &= b ? bal : ~bal;
    }
    const int rank = __popcll(same & lt);
    const int cnt = __popcll(same);
    if (valid && rank == 0) wcnt[w][e] = cnt;
    __syncthreads();
    if (valid) {
      int pos = running[e] + rank;
      for (int v = 0; v < w; ++v) pos += wcnt[v][e];
      sorted_pair[pos] = (int32_t)f;
      inv_pos[f] = pos;
    } else if (in) {
      inv_pos[f] = -1;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&running[e], cnt);
      wcnt[w][e] = 0;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- tile lists
// List b of the plan from the expert offsets, by one workgroup of 256
// threads: per-expert tile counts (thread t takes experts [4t, 4t + 4)),
// their exclusive scan, then tile t to thread t mod 256, which finds its
// expert by binary search over the experts' first tiles in LDS, so the time
// does not depend on how the rows are spread over the experts.  Tiles come
// out expert-major (the order of the oracle's lists).  lds: 3 kMaxExperts ints.
constexpr int kListEPT = kMaxExperts / 256;
__device__ __forceinline__ void write_list(int b, const int32_t* __restrict__ offsets, int slots,
                                           int32_t* __restrict__ plan, int list_off, int* lds) {
  int* const first = lds;
  int* const e_start = lds + kMaxExperts;
  int* const e_rows = lds + 2 * kMaxExperts;
  __shared__ int wsum[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, BM = kPlanBMs[b];
  int nt[kListEPT], st[kListEPT], nr[kListEPT];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kListEPT; ++k) {
    const int e = t * kListEPT + k;
    st[k] = e < slots ? offsets[e] : 0;
    nr[k] = e < slots ? offsets[e + 1] - st[k] : 0;
    nt[k] = (e < slots && plan_list_has(b, nr[k])) ? (nr[k] + BM - 1) / BM : 0;
    sum += nt[k];
  }
  int x = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int run = x - sum, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += i < w ? wsum[i] : 0;
    total += wsum[i];
  }
#pragma unroll
  for (int k = 0; k < kListEPT; ++k) {
    const int e = t * kListEPT + k;
    if (e < slots) {
      first[e] = run;
      e_start[e] = st[k];
      e_rows[e] = nr[k];
    }
    run += nt[k];
  }
  if (t == 0) {
    plan[b] = total;
    plan[kPlanLists + b] = list_off;
  }
  __syncthreads();
  for (int tt = t; tt < total; tt += 256) {
    // The last expert whose first tile is <= tt owns tile tt (an expert
    // with no tile here shares its first index with the next expert).
    int l = 0, h = slots - 1;
    while (l < h) {
      const int mid = (l + h + 1) >> 1;
      if (first[mid] <= tt) l = mid;
      else h = mid - 1;
    }
    write_tile(plan + list_off + 2 * tt, l, tt - first[l], BM, e_start[l], e_rows[l]);
  }
}

// ---------------------------------------------------------------- one workgroup
// The whole alignment in one launch when P <= kSmallP (at most 4 pairs per
// thread).  LDS atomics count the pairs of every expert and hand each pair a
// slot in its expert's segment, in arbitrary order; after the scan over
// experts the pair indices are placed there, and each pair's final row is its
// segment start plus the number of smaller pair indices in the segment -- a
// stable order that no atomic ordering can change.  Each thread then writes
// only its own pairs.
constexpr int kSmallP = 4096;
constexpr int kSmallPer = kSmallP / 1024;

// Dense use (no ids, one expert): the identity permutation and the tile
// lists of one expert with P rows, written directly (no counting, no scans).
__device__ __forceinline__ void dense_plan_body(const AlignP& a, int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ sorted_pair,
                                                int32_t* __restrict__ inv_pos,
                                                int32_t* __restrict__ plan, PlanOffs list_off) {
  const int P = (int)a.P, tid = threadIdx.x;
  for (int f = tid; f < P; f += blockDim.x) {
    sorted_pair[f] = f;
    inv_pos[f] = f;
  }
#pragma unroll
  for (int b = 0; b < kPlanLists; ++b) {
    const int n_t = plan_list_has(b, P) ? (P + kPlanBMs[b] - 1) / kPlanBMs[b] : 0;
    for (int mt = tid; mt < n_t; mt += blockDim.x)
      write_tile(plan + list_off.v[b] + 2 * mt, 0, mt, kPlanBMs[b], 0, P);
    if (tid == 0) {
      plan[b] = n_t;
      plan[kPlanLists + b] = list_off.v[b];
    }
  }
  if (tid == 0) {
    offsets[0] = 0;
    offsets[1] = P;
  }
}

__device__ __forceinline__ void align_small_body(const AlignP& a, int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ sorted_pair,
                                                 int32_t* __restrict__ inv_pos,
                                                 int32_t* __restrict__ plan, PlanOffs list_off) {
  if (a.ids == nullptr && a.slots == 1) {
    dense_plan_body(a, offsets, sorted_pair, inv_pos, plan, list_off);
    return;
  }
  __shared__ int cnt[kMaxExperts];
  __shared__ int running[kMaxExperts];
  __shared__ int wcnt[16][kMaxExperts];   // pairs of an expert per wavefront, current round
  const int tid = threadIdx.x;
  const int P = (int)a.P;
  for (int x = tid; x < a.slots; x += 1024) cnt[x] = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    for (int x = tid; x < a.slots; x += 1024) wcnt[v][x] = 0;
  __syncthreads();
  int my_e[kSmallPer];
#pragma unroll
  for (int r = 0; r < kSmallPer; ++r) {
    const int f = tid + 1024 * r;
    my_e[r] = -1;
    if (f < P) {
      bool valid;
      const int e = expert_of(a, f, valid);
      if (valid) {
        my_e[r] = e;
        atomicAdd(&cnt[e], 1);
      } else {
        inv_pos[f] = -1;
      }
    }
  }
  __syncthreads();
  const int e = tid;
  const int n_e = e < a.slots ? cnt[e] : 0;
  int pk[3];
  plan_counts_small(e, a.slots, n_e, pk);
  const int sv[4] = {n_e, pk[0], pk[1], pk[2]};
  int sx[4], st[4];
  block_exclusive_scan_1024_v<4>(sv, sx, st);
  const int off_e = sx[0], total = st[0];
  write_plan_small(plan, list_off, e, a.slots, off_e, n_e, {sx[1], sx[2], sx[3]}, {st[1], st[2], st[3]});
  if (e < a.slots) {
    offsets[e] = off_e;
    running[e] = off_e;
  }
  if (e == 0) offsets[a.slots] = total;
  __syncthreads();
  // Stable order without comparisons: in round r the 1024 pairs
  // f = 1024 r + tid are in increasing order, so a pair's row is its
  // expert's rows of the earlier rounds (running), plus those of the earlier
  // wavefronts of this round (wcnt), plus the lower lanes of its own
  // wavefront with the same expert (an 11-bit ballot match).
  const int w = tid >> 6, lane = tid & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kSmallPer; ++r) {
    if (1024 * r >= P) break;  // (uniform: rounds past the last pair)
    const int ex = my_e[r];
    const bool valid = ex >= 0;
    const int key = valid ? ex : 2047;
    uint64_t same = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) {
      const bool bb = (key >> bit) & 1;
      const uint64_t bal = __ballot(bb);
      same &= bb ? bal : ~bal;
    }
    const int rank = __popcll(same & lt);
    const int cw = __popcll(same);
    if (valid && rank == 0) wcnt[w][ex] = cw;
    __syncthreads();
    if (valid) {
      int pos = running[ex] + rank;
      for (int v = 0; v < w; ++v) pos += wcnt[v][ex];
      const int f = tid + 1024 * r;
      sorted_pair[pos] = f;
      inv_pos[f] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&running[ex], cw);
      wcnt[w][ex] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(1024) void align_small_kernel(AlignP a, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ inv_pos,
                                                           int32_t* __restrict__ plan, PlanOffs list_off) {
  align_small_body(a, offsets, sorted_pair, inv_pos, plan, list_off);
}

// ---------------------------------------------------------------- scale + align
// The activation global scale and the alignment are independent: one launch
// runs both.  Workgroups 0 .. nblk-1 reduce max |x| over the bf16 tensor
// (each folds its maximum into ws[1] and counts itself in ws[0]; the last one
// writes g and puts both words back to zero, as nvfp4_global_scale does) and
// workgroup nblk runs the one-workgroup alignment.
__global__ __launch_bounds__(1024) void scale_align_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                           float* __restrict__ g,
                                                           uint32_t* __restrict__ ws, int nblk,
                                                           AlignP a, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ inv_pos,
                                                           int32_t* __restrict__ plan, PlanOffs list_off) {
  if ((int)blockIdx.x == nblk) {
    align_small_body(a, offsets, sorted_pair, inv_pos, plan, list_off);
    return;
  }
  __shared__ float red[16];
  const int64_t stride = (int64_t)nblk * 1024 * 8;
  float m = 0.0f;
  // U independent loads per trip (the grid gives each thread about 4).
  constexpr int U = 4;
  int64_t i = ((int64_t)blockIdx.x * 1024 + threadIdx.x) * 8;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const u32x4*>(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = fmaxf(m, amax_input(bf16_bits_to_f32(w[u][j] & 0xFFFFu)));
        m = fmaxf(m, amax_input(bf16_bits_to_f32(w[u][j] >> 16)));
      }
  }
  for (; i < n; i += stride) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(x + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, amax_input(bf16_bits_to_f32(w[j] & 0xFFFFu)));
      m = fmaxf(m, amax_input(bf16_bits_to_f32(w[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x != 0) return;
  float r = red[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) r = fmaxf(r, red[i]);
  if (nblk == 1) {
    *g = global_scale_of_amax(r);
    return;
  }
  fold_max_and_count(ws, ws + 1, r, (uint32_t)nblk, g);
}

// ---------------------------------------------------------------- large batches
// Global scale, quantisation and alignment beyond the single fused launch
// (P > kSmallP, or T*H > kFusedQuantMax): three launches instead of the
// five of the separate steps (scale, count, scan, scatter, quantise), and no
// cross-workgroup atomics.
//   1. scale_count_kernel: workgroups [0, nb) each store max |x| over their
//      share of the tensor in partial[b]; workgroups [nb, nb + nchunks) each
//      count the experts of one pair chunk.
//   2. scan_scale_kernel: the one-workgroup scan (chunk bases and expert
//      offsets), which also takes the maximum of the nb partial maxima and
//      writes g.
//   3. scatter_plan_quant_kernel: workgroups [0, nchunks) place the pairs
//      of one chunk, the next six write one tile list each, the others
//      quantise x with g.
// A maximum is exact in any grouping, so g is bit for bit the one of the
// single-launch reduction (nvfp4_global_scale).
constexpr int kScalePartials = 1024;  // most workgroups of the fused global scale
constexpr int kScaleThreads = 256;
constexpr int kScaleLoads = 8;   // 16-byte loads per thread and trip

__global__ __launch_bounds__(kScaleThreads) void scale_count_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                    int nb, float* __restrict__ partial,
                                                                    AlignP a, int32_t* __restrict__ counts) {
  if ((int)blockIdx.x >= nb) {
    count_chunk(a, counts, (int)blockIdx.x - nb);
    return;
  }
  __shared__ float red[kScaleThreads / 64];
  constexpr int U = kScaleLoads;
  const int64_t stride = (int64_t)nb * kScaleThreads * 8;
  float m = 0.0f;
  int64_t i = ((int64_t)blockIdx.x * kScaleThreads + threadIdx.x) * 8;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const u32x4*>(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = fmaxf(m, amax_input(bf16_bits_to_f32(w[u][j] & 0xFFFFu)));
        m = fmaxf(m, amax_input(bf16_bits_to_f32(w[u][j] >> 16)));
      }
  }
  for (; i < n; i += stride) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(x + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, amax_input(bf16_bits_to_f32(w[j] & 0xFFFFu)));
      m = fmaxf(m, amax_input(bf16_bits_to_f32(w[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int k = 1; k < kScaleThreads / 64; ++k) r = fmaxf(r, red[k]);
    partial[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(1024) void scan_scale_kernel(AlignP a, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          const float* __restrict__ partial, int nb,
                                                          float* __restrict__ g) {
  // (requested first, so its latency overlaps the scan's own loads)
  float m = (int)threadIdx.x < nb ? partial[threadIdx.x] : 0.0f;
  scan_body(a, counts, offsets);
  __shared__ float red[16];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) r = fmaxf(r, red[k]);
    *g = global_scale_of_amax(r);
  }
}

// Workgroups [0, nchunks): the pairs of one chunk; the next kPlanLists: one
// tile list each; the rest (if x): quantisation of x -- NVFP4 with g (q
// codes, sf E4M3 scales, optional x_deq), one lane per 16-element block
// (BLOCK) or per 8 elements, or (MX) OCP MXFP4, one lane per 8 elements (q
// codes, sf E8M0 bytes).  The roles share one LDS area.
template <bool MX, bool BLOCK>
__global__ __launch_bounds__(256) void scatter_plan_quant_kernel(
    AlignP a, const int32_t* __restrict__ bases, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ inv_pos, const int32_t* __restrict__ offsets, int32_t* __restrict__ plan,
    PlanOffs list_off, const uint16_t* __restrict__ x, uint32_t n_hb, uint32_t hb_per_row, int64_t H,
    const float* __restrict__ g, uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
    uint16_t* __restrict__ x_deq) {
  __shared__ int lds[kScatterLds];
  const int blk = (int)blockIdx.x;
  if (blk < a.nchunks) {
    scatter_chunk(a, bases, sorted_pair, inv_pos, blk, lds);
    return;
  }
  if (blk < a.nchunks + kPlanLists) {
    const int b = blk - a.nchunks;
    write_list(b, offsets, a.slots, plan, list_off.v[b], lds);
    return;
  }
  const uint32_t i = ((uint32_t)blk - (uint32_t)(a.nchunks + kPlanLists)) * 256u + threadIdx.x;
  if constexpr (!MX && BLOCK) {
    // NVFP4, block i (16 elements) per lane.  32-bit indices: n_hb < 2^31
    // (checked by the launcher).
    const uint32_t b_per_row = hb_per_row >> 1;
    if (i >= (n_hb >> 1)) return;
    const uint32_t row = i / b_per_row;
    quantize_block(x, (int64_t)row, (int64_t)(i - row * b_per_row) << 4, H, H, ld_uniform(g), q, sf, x_deq);
  } else {
    // Half-block i (8 elements); the lanes of a block (2 for NVFP4, 4 for
    // MXFP4) take the same branch (n_hb is a multiple of 4).
    if (i >= n_hb) return;
    float v[8];
    load8(x, (int64_t)i * 8, v);
    const uint32_t row = i / hb_per_row;
    const int64_t c8 = (int64_t)(i - row * hb_per_row) << 3;
    if constexpr (MX)
      mx_quantize8_canonical(v, (int64_t)row, c8, H, q, sf);
    else
      quantize_half_block_values(v, (int64_t)row, c8, H, ld_uniform(g), q, sf, x_deq);
  }
}

// OCP MXFP4 quantisation and alignment in one launch when the pairs fit one
// workgroup: workgroups 0 .. nblk-1 quantise (grid-strided; the four lanes
// of a 32-element block stay together), workgroup nblk runs the
// one-workgroup alignment.  The two are independent (no global scale).
__global__ __launch_bounds__(1024) void mx_quant_align_kernel(const uint16_t* __restrict__ x, uint32_t n_hb,
                                                              uint32_t hb_per_row, int64_t H,
                                                              uint8_t* __restrict__ q, uint8_t* __restrict__ ex,
                                                              int nblk, AlignP a, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_pair,
                                                              int32_t* __restrict__ inv_pos,
                                                              int32_t* __restrict__ plan, PlanOffs list_off) {
  if ((int)blockIdx.x == nblk) {
    align_small_body(a, offsets, sorted_pair, inv_pos, plan, list_off);
    return;
  }
  for (uint32_t i = blockIdx.x * 1024u + threadIdx.x; i < n_hb; i += (uint32_t)nblk * 1024u) {
    float v[8];
    load8(x, (int64_t)i * 8, v);
    const uint32_t row = i / hb_per_row;
    mx_quantize8_canonical(v, (int64_t)row, (int64_t)(i - row * hb_per_row) << 3, H, q, ex);
  }
}

// ---------------------------------------------------------------- quantise + align
// Activation global scale, NVFP4 quantisation and alignment in one launch,
// for decode-sized activations.  Workgroups 0 .. nblk-1 each reduce max |x|
// over the whole tensor (small enough to come from L2; the maximum is exact,
// so all of them find the same g) and then quantise their share of the
// 8-element half-blocks; workgroup nblk runs the one-workgroup alignment.
// No workgroup waits for another.
constexpr int64_t kFusedQuantMax = int64_t(1) << 18;  // elements of x

__global__ __launch_bounds__(1024) void quant_align_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                           int64_t H, float* __restrict__ g,
                                                           uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ sf,
                                                           uint16_t* __restrict__ x_deq, int nblk,
                                                           AlignP a, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ inv_pos,
                                                           int32_t* __restrict__ plan, PlanOffs list_off) {
  if ((int)blockIdx.x == nblk) {
    align_small_body(a, offsets, sorted_pair, inv_pos, plan, list_off);
    return;
  }
  __shared__ float red[16];
  const int64_t n = T * H;
  float m = 0.0f;
  // 16 independent loads per trip, one trip at T*H = 2^17 (indices past
  // the end are clamped to the last 8 elements: re-reading them cannot change
  // a maximum).  For bf16 values that are not NaN, |x| orders like the
  // unsigned 15-bit pattern, so the maximum is taken on packed 16-bit
  // integers.  NaN patterns (above 0x7F80) are cleared first, so that a NaN
  // takes no part in the maximum, as in fmaxf of the unfused reduction: the
  // two dispatch paths give the same g for every input.
  constexpr int U = 16;
  u16x2 mm = {0, 0};
  for (int64_t base = (int64_t)threadIdx.x * 8; base < n; base += U * 1024 * 8) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = *reinterpret_cast<const u32x4*>(x + min(base + (int64_t)u * 1024 * 8, n - 8));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mag = w[u][j] & 0x7FFF7FFFu;
        // Bit 15 of a half is set by the addition exactly when that half
        // exceeds 0x7F80 (no carry crosses halves: each stays below 2^16).
        const uint32_t nan = ((mag + 0x007F007Fu) & 0x80008000u) >> 15;
        mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, mag & ~(nan * 0xFFFFu)));
      }
  }
  m = bf16_bits_to_f32(max((uint32_t)mm[0], (uint32_t)mm[1]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) r = fmaxf(r, red[i]);
  const float gv = global_scale_of_amax(r);
  if (blockIdx.x == 0 && threadIdx.x == 0) *g = gv;
  // Half-blocks i (8 elements); both lanes of a block have the same trip
  // count because n / 8 is even (H is a multiple of 128).
  // 32-bit index arithmetic (n <= kFusedQuantMax): the row division is the
  // costliest step of the loop in 64 bits.
  static_assert(kFusedQuantMax / 8 < (int64_t(1) << 31), "half-block indices fit 32 bits");
  const uint32_t hb_per_row = (uint32_t)(H >> 3), n_hb = (uint32_t)(n / 8);
  for (uint32_t i = blockIdx.x * 1024u + threadIdx.x; i < n_hb; i += (uint32_t)nblk * 1024u) {
    const uint32_t row = i / hb_per_row;
    float v[8];
    load8(x, (int64_t)i * 8, v);
    quantize_half_block_values(v, (int64_t)row, (int64_t)(i - row * hb_per_row) << 3, H, gv, q, sf, x_deq);
  }
}

// ---------------------------------------------------------------- router
// One wavefront per token: k rounds of (max logit, lowest id) selection.
// One wavefront routes token t: k rounds of (max logit, lowest id) over the
// E logits (16 per lane), then the softmax over the selected logits in FP64.
// sel_v / sel_i: this wavefront's 32-entry LDS scratch.
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ wts,
                                            float* sel_v, int* sel_i, double* sel_e) {
  const int lane = threadIdx.x & 63;
  const float* z = logits + (int64_t)t * E;
  float v[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = lane + 64 * i;
    v[i] = idx < E ? z[idx] : -INFINITY;
    if (idx >= E) taken |= 1u << i;
  }
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !((taken >> i) & 1u);
      const bool better = ok && (v[i] > bv || (v[i] == bv && lane + 64 * i < bi));
      bv = better ? v[i] : bv;
      bi = better ? lane + 64 * i : bi;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const bool better = ov > bv || (ov == bv && oi < bi);
      bv = better ? ov : bv;
      bi = better ? oi : bi;
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      sel_v[j] = bv;
      sel_i[j] = bi;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  // Each selected exponential once (lane j), then the same sequential sum
  // in every lane.
  double mine = 0.0;
  if (lane < k) {
    mine = exp((double)sel_v[lane] - (double)sel_v[0]);
    sel_e[lane] = mine;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  if (lane < k) {
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += sel_e[j];
    ids[(int64_t)t * k + lane] = sel_i[lane];
    wts[(int64_t)t * k + lane] = (float)(mine / sum);
  }
  // (the next token of this wavefront rewrites sel_v / sel_i only after all
  // lanes have read them)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
// One (value, index) step of the row reduction: keep the larger logit, the
// lower id on equal logits.
template <int CTRL>
__device__ __forceinline__ void route_step(float& bv, int& bi) {
  const float ov = __int_as_float(dpp_i<CTRL>(__float_as_int(bv)));
  const int oi = dpp_i<CTRL>(bi);
  const bool better = ov > bv || (ov == bv && oi < bi);
  bv = better ? ov : bv;
  bi = better ? oi : bi;
}

// The same selection by one 16-lane DPP row per token (E <= 256: logit
// r + 16 i in lane r), so a wavefront routes 4 tokens at once and each of the
// k rounds reduces over the row with 4 DPP steps.  Same choices and the same
// FP64 softmax as route_token.
__device__ __forceinline__ void route_token16(const float* __restrict__ logits, int t, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ wts,
                                              float* sel_v, int* sel_i, double* sel_e) {
  const int r = threadIdx.x & 15;
  const float* z = logits + (int64_t)t * E;
  float v[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = r + 16 * i;
    v[i] = idx < E ? z[idx] : -INFINITY;
    if (idx >= E) taken |= 1u << i;
  }
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !((taken >> i) & 1u);
      const bool better = ok && (v[i] > bv || (v[i] == bv && r + 16 * i < bi));
      bv = better ? v[i] : bv;
      bi = better ? r + 16 * i : bi;
    }
    route_step<0xB1>(bv, bi);   // lane ^ 1
    route_step<0x4E>(bv, bi);   // lane ^ 2
    route_step<0x141>(bv, bi);  // half-row mirror
    route_step<0x140>(bv, bi);  // row mirror
    if ((bi & 15) == r) taken |= 1u << (bi >> 4);
    if (r == 0) {
      sel_v[j] = bv;
      sel_i[j] = bi;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  // Each selected exponential once (lane j % 16), then the same sequential
  // sum as route_token.
  for (int jj = r; jj < k; jj += 16) sel_e[jj] = exp((double)sel_v[jj] - (double)sel_v[0]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  if (r < k) {
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += sel_e[j];
    for (int jj = r; jj < k; jj += 16) {
      ids[(int64_t)t * k + jj] = sel_i[jj];
      wts[(int64_t)t * k + jj] = (float)(sel_e[jj] / sum);
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
  __shared__ float sel_v[4][32];
  __shared__ int sel_i[4][32];
  __shared__ double sel_e[4][32];
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  route_token(logits, t, E, k, ids, wts, sel_v[w], sel_i[w], sel_e[w]);
}

// 16 tokens per workgroup, one per 16-lane row (E <= 256).
__global__ __launch_bounds__(256) void route_topk16_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int32_t* __restrict__ ids,
                                                           float* __restrict__ wts) {
  __shared__ float sel_v[16][32];
  __shared__ int sel_i[16][32];
  __shared__ double sel_e[16][32];
  const int g = threadIdx.x >> 4;
  const int t = blockIdx.x * 16 + g;
  if (t >= T) return;   // whole rows leave together
  route_token16(logits, t, E, k, ids, wts, sel_v[g], sel_i[g], sel_e[g]);
}

}  // namespace

AlignShape align_shape(int T, int topk, int E, int shared) {
  AlignShape a;
  a.T = T;
  a.topk = topk;
  a.E = E;
  a.shared = shared;
  a.H = 0;
  a.P = (int64_t)T * topk + (int64_t)shared * T;
  a.slots = E + shared;
  a.nchunks = (int)((a.P + kAlignChunk - 1) / kAlignChunk);
  int64_t off = kPlanHeader;
  for (int b = 0; b < kPlanLists; ++b) {
    a.list_off[b] = off;
    // Every expert adds at most one partial tile; list 5 holds only experts
    // with more than kSplitRows rows, of which there are at most P / (kSplitRows + 1).
    const int64_t experts = b == 5 ? std::min<int64_t>(a.slots, a.P / (kSplitRows + 1)) : a.slots;
    a.list_len[b] = (a.P + kPlanBMs[b] - 1) / kPlanBMs[b] + experts;
    off += 2 * a.list_len[b];
  }
  return a;
}

size_t align_ws_bytes(const AlignShape& a) {
  // per-chunk expert counts, then the partial maxima of the fused global
  // scale (moe_quantize_and_align beyond one launch)
  return (size_t)a.nchunks * (size_t)a.slots * sizeof(int32_t) + (size_t)kScalePartials * sizeof(float);
}

size_t align_plan_ints(const AlignShape& a) {
  return (size_t)(a.list_off[kPlanLists - 1] + 2 * a.list_len[kPlanLists - 1]);
}

PlanOffs plan_offsets(const AlignShape& a) {
  PlanOffs o;
  for (int b = 0; b < kPlanLists; ++b) o.v[b] = (int)a.list_off[b];
  return o;
}

hipError_t launch_align(const AlignShape& a, const int32_t* topk_ids, int32_t* offsets,
                        int32_t* sorted_pair, int32_t* inv_pos, int32_t* plan, void* ws,
                        hipStream_t s) {
  AlignP p;
  p.ids = topk_ids;
  p.T = a.T;
  p.topk = a.topk;
  p.E = a.E;
  p.shared = a.shared;
  p.slots = a.slots;
  p.nchunks = a.nchunks;
  p.P = a.P;
  int32_t* counts = static_cast<int32_t*>(ws);
  const PlanOffs lo0 = plan_offsets(a);
  if (a.P <= (int64_t)kSmallP) {
    align_small_kernel<<<1, 1024, 0, s>>>(p, offsets, sorted_pair, inv_pos, plan, lo0);
    return hipGetLastError();
  }
  if (a.nchunks > 0) {
    align_count_kernel<<<a.nchunks, 256, 0, s>>>(p, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const PlanOffs lo = plan_offsets(a);
  align_scan_kernel<<<1, 1024, 0, s>>>(p, counts, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the pair scatter beside the six tile lists
  scatter_plan_quant_kernel<false, false><<<a.nchunks + kPlanLists, 256, 0, s>>>(
      p, counts, sorted_pair, inv_pos, offsets, plan, lo, nullptr, 0u, 1u, 0, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_scale_and_align(const AlignShape& a, const uint16_t* x, float* g, void* gs_ws,
                                  const int32_t* topk_ids, int32_t* offsets, int32_t* sorted_pair,
                                  int32_t* inv_pos, int32_t* plan, void* ws, hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.H;
  if (a.P > (int64_t)kSmallP || n == 0) {
    hipError_t e = launch_global_scale(x, 0, 1, n, g, gs_ws, s);
    if (e != hipSuccess) return e;
    return launch_align(a, topk_ids, offsets, sorted_pair, inv_pos, plan, ws, s);
  }
  AlignP p;
  p.ids = topk_ids;
  p.T = a.T;
  p.topk = a.topk;
  p.E = a.E;
  p.shared = a.shared;
  p.slots = a.slots;
  p.nchunks = a.nchunks;
  p.P = a.P;
  int nblk = (int)((n + 1024 * 32 - 1) / (1024 * 32));
  nblk = nblk < 1 ? 1 : (nblk > 256 ? 256 : nblk);
  const PlanOffs lo = plan_offsets(a);
  scale_align_kernel<<<nblk + 1, 1024, 0, s>>>(x, n, g, static_cast<uint32_t*>(gs_ws), nblk, p, offsets,
                                               sorted_pair, inv_pos, plan, lo);
  return hipGetLastError();
}

hipError_t launch_quantize_and_align(const AlignShape& a, const uint16_t* x, float* g, void* gs_ws,
                                    uint8_t* q, uint8_t* sf, uint16_t* x_deq,
                                    const int32_t* topk_ids, int32_t* offsets, int32_t* sorted_pair,
                                    int32_t* inv_pos, int32_t* plan, void* ws, hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.H;
  // Beyond the single fused launch (P > kSmallP or T*H > kFusedQuantMax):
  // three launches (at the 512-expert layer's 2816 pairs and 2^20 elements,
  // 2 us faster than the global scale + one-workgroup alignment launch
  // followed by the quantisation).  Dense use (no ids, one expert) keeps the
  // alignment's direct identity plan when it fits one workgroup.
  const bool dense = topk_ids == nullptr && a.slots == 1;
  if ((a.P > (int64_t)kSmallP || (n > kFusedQuantMax && !dense)) && n > 0 && n / 8 < (int64_t(1) << 31)) {
    AlignP p;
    p.ids = topk_ids;
    p.T = a.T;
    p.topk = a.topk;
    p.E = a.E;
    p.shared = a.shared;
    p.slots = a.slots;
    p.nchunks = a.nchunks;
    p.P = a.P;
    int32_t* counts = static_cast<int32_t*>(ws);
    float* partial = reinterpret_cast<float*>(counts + (int64_t)a.nchunks * a.slots);
    // one trip of kScaleLoads loads per thread when the tensor allows
    const int64_t per_blk = (int64_t)kScaleThreads * 8 * kScaleLoads;
    const int nb = (int)std::min<int64_t>(kScalePartials, std::max<int64_t>(1, (n + per_blk - 1) / per_blk));
    scale_count_kernel<<<nb + a.nchunks, kScaleThreads, 0, s>>>(x, n, nb, partial, p, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    scan_scale_kernel<<<1, 1024, 0, s>>>(p, counts, offsets, partial, nb, g);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_hb = n / 8;
    // a lane per 16-element block from 2^18 blocks, else per 8 elements
    // (as nvfp4_quantize)
    const bool block = n_hb / 2 >= (int64_t(1) << 18);
    const int64_t qblocks = ((block ? n_hb / 2 : n_hb) + 255) / 256;
    const unsigned grid = (unsigned)(a.nchunks + kPlanLists + qblocks);
    if (block)
      scatter_plan_quant_kernel<false, true><<<grid, 256, 0, s>>>(p, counts, sorted_pair, inv_pos, offsets, plan,
                                                                  plan_offsets(a), x, (uint32_t)n_hb,
                                                                  (uint32_t)(a.H >> 3), a.H, g, q, sf, x_deq);
    else
      scatter_plan_quant_kernel<false, false><<<grid, 256, 0, s>>>(p, counts, sorted_pair, inv_pos, offsets, plan,
                                                                   plan_offsets(a), x, (uint32_t)n_hb,
                                                                   (uint32_t)(a.H >> 3), a.H, g, q, sf, x_deq);
    return hipGetLastError();
  }
  if (a.P > (int64_t)kSmallP || n == 0 || n > kFusedQuantMax) {
    hipError_t e = launch_scale_and_align(a, x, g, gs_ws, topk_ids, offsets, sorted_pair, inv_pos, plan,
                                          ws, s);
    if (e != hipSuccess) return e;
    return launch_quantize(x, 0, a.T, a.H, a.H, g, a.T, q, sf, x_deq, s);
  }
  AlignP p;
  p.ids = topk_ids;
  p.T = a.T;
  p.topk = a.topk;
  p.E = a.E;
  p.shared = a.shared;
  p.slots = a.slots;
  p.nchunks = a.nchunks;
  p.P = a.P;
  const int nblk = (int)((n / 8 + 1023) / 1024);  // 1 .. 32
  const PlanOffs lo = plan_offsets(a);
  quant_align_kernel<<<nblk + 1, 1024, 0, s>>>(x, a.T, a.H, g, q, sf, x_deq, nblk, p, offsets, sorted_pair,
                                               inv_pos, plan, lo);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_and_align(const AlignShape& a, const uint16_t* x, uint8_t* q, uint8_t* ex,
                                       const int32_t* topk_ids, int32_t* offsets, int32_t* sorted_pair,
                                       int32_t* inv_pos, int32_t* plan, void* ws, hipStream_t s) {
  AlignP p;
  p.ids = topk_ids;
  p.T = a.T;
  p.topk = a.topk;
  p.E = a.E;
  p.shared = a.shared;
  p.slots = a.slots;
  p.nchunks = a.nchunks;
  p.P = a.P;
  const int64_t n_hb = (int64_t)a.T * a.H / 8;
  const PlanOffs lo = plan_offsets(a);
  if (a.P <= (int64_t)kSmallP) {
    const int nblk = (int)std::min<int64_t>(256, std::max<int64_t>(1, (n_hb + 1023) / 1024));
    mx_quant_align_kernel<<<nblk + 1, 1024, 0, s>>>(x, (uint32_t)n_hb, (uint32_t)(a.H >> 3), a.H, q, ex, nblk, p,
                                                     offsets, sorted_pair, inv_pos, plan, lo);
    return hipGetLastError();
  }
  int32_t* counts = static_cast<int32_t*>(ws);
  align_count_kernel<<<a.nchunks, 256, 0, s>>>(p, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  align_scan_kernel<<<1, 1024, 0, s>>>(p, counts, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t qblocks = (n_hb + 255) / 256;   // one lane per 8 elements
  scatter_plan_quant_kernel<true, false><<<(unsigned)(a.nchunks + kPlanLists + qblocks), 256, 0, s>>>(
      p, counts, sorted_pair, inv_pos, offsets, plan, lo, x, (uint32_t)n_hb, (uint32_t)(a.H >> 3), a.H, nullptr,
      q, ex, nullptr);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  if (E <= 256)
    route_topk16_kernel<<<(T + 15) / 16, 256, 0, s>>>(logits, T, E, k, ids, w);
  else
    route_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_route_and_align(const AlignShape& a, const float* logits, int32_t* ids, float* w,
                                  int32_t* offsets, int32_t* sorted_pair, int32_t* inv_pos,
                                  int32_t* plan, void* ws, hipStream_t s) {
  // Two launches: routing is a latency chain per token (k rounds of a
  // reduction), and one workgroup holding both steps (all tokens on one CU)
  // measured slower than the router's own grid followed by the alignment.
  if (a.T > 0) {
    hipError_t e = launch_route_topk(logits, a.T, a.E, a.topk, ids, w, s);
    if (e != hipSuccess) return e;
  }
  return launch_align(a, ids, offsets, sorted_pair, inv_pos, plan, ws, s);
}

}  // namespace nvfp4
