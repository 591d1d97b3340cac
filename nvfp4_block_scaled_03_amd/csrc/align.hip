// Router and permutation by expert (gfx950).
//
// moe_align groups the (token, expert) pairs by expert with a stable order --
// the grouped-GEMM metadata step (get_cutlass_moe_mm_data) of vLLM PR #29242
// -- without atomics deciding any position: per-chunk histograms, a per-expert
// scan, then a scatter whose in-chunk ranks come from wavefront ballots.  It
// also writes the tile lists the grouped GEMMs read, so per-expert problem
// sizes never leave the device (vLLM PR #29242, debug trace: the host problem
// shape is not available to the grouped GEMM).
#include "common.h"
#include "launch.h"

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
    const int e = a.ids[f];
    valid = e >= 0 && e < a.E;
    return e;
  }
  valid = true;
  return a.E;  // shared expert slot
}

// ---------------------------------------------------------------- counts
__global__ __launch_bounds__(256) void align_count_kernel(AlignP a, int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < a.slots; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)blockIdx.x * kAlignChunk;
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
    counts[(int64_t)blockIdx.x * a.slots + e] = hist[e];
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
__device__ __forceinline__ void write_tile(int32_t* dst, int e, int mt, int BM, const int* soff) {
  const int row0 = soff[e] + mt * BM;
  const int rows = min(BM, soff[e + 1] - row0);
  dst[0] = e | (mt << 11);
  dst[1] = (int32_t)((uint32_t)row0 | ((uint32_t)rows << 24));
}

// ---------------------------------------------------------------- scan + plan
__global__ __launch_bounds__(1024) void align_scan_kernel(AlignP a, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ plan,
                                                          int4 list_off) {
  __shared__ int tstart[kMaxExperts + 1];
  __shared__ int soff[kMaxExperts + 1];
  const int e = threadIdx.x;
  int n_e = 0;
  if (e < a.slots) {
    for (int c = 0; c < a.nchunks; ++c) {
      const int64_t i = (int64_t)c * a.slots + e;
      const int v = counts[i];
      counts[i] = n_e;  // exclusive prefix over earlier chunks
      n_e += v;
    }
  }
  int total;
  const int off_e = block_exclusive_scan_1024(n_e, &total);
  if (e < a.slots) {
    for (int c = 0; c < a.nchunks; ++c) counts[(int64_t)c * a.slots + e] += off_e;
    offsets[e] = off_e;
    soff[e] = off_e;
  }
  if (e == 0) {
    offsets[a.slots] = total;
    soff[a.slots] = total;
  }

  const int lo[4] = {list_off.x, list_off.y, list_off.z, list_off.w};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int BM = kPlanBMs[b];
    const int tiles = (e < a.slots) ? (n_e + BM - 1) / BM : 0;
    int ntiles;
    const int ts = block_exclusive_scan_1024(tiles, &ntiles);
    if (e < a.slots) tstart[e] = ts;
    if (e == 0) {
      tstart[a.slots] = ntiles;
      plan[b] = ntiles;
      plan[4 + b] = lo[b];
    }
    __syncthreads();
    for (int slot = threadIdx.x; slot < ntiles; slot += 1024) {
      // largest expert x with tstart[x] <= slot
      int l = 0, h = a.slots;  // tstart[l] <= slot < tstart[h]
      while (h - l > 1) {
        const int m = (l + h) >> 1;
        if (tstart[m] <= slot) l = m; else h = m;
      }
      write_tile(plan + lo[b] + 2 * slot, l, slot - tstart[l], BM, soff);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- scatter
__global__ __launch_bounds__(256) void align_scatter_kernel(AlignP a,
                                                            const int32_t* __restrict__ bases,
                                                            int32_t* __restrict__ sorted_pair,
                                                            int32_t* __restrict__ inv_pos) {
  __shared__ int running[kMaxExperts];
  __shared__ int wcnt[4][kMaxExperts];
  for (int e = threadIdx.x; e < a.slots; e += 256) {
    running[e] = bases[(int64_t)blockIdx.x * a.slots + e];
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kAlignChunk / 256; ++r) {
    const int64_t f = (int64_t)blockIdx.x * kAlignChunk + r * 256 + threadIdx.x;
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

// ---------------------------------------------------------------- one workgroup
// The whole alignment in one launch when P <= 4 * kAlignChunk: histogram,
// scan, tile lists and the stable scatter, by 1024 threads in rounds of 1024
// pairs (the in-round order of equal experts comes from wavefront ballots and
// per-wavefront counts, as in the multi-workgroup path).
constexpr int kFusedRounds = 4;

__global__ __launch_bounds__(1024) void align_fused_kernel(AlignP a, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ inv_pos,
                                                           int32_t* __restrict__ plan, int4 list_off) {
  __shared__ int hist[kMaxExperts];
  __shared__ int running[kMaxExperts];
  __shared__ int tstart[kMaxExperts + 1];
  __shared__ int soff[kMaxExperts + 1];
  __shared__ int wcnt[16][kMaxExperts];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (tid < a.slots) hist[tid] = 0;
  for (int i = tid; i < 16 * kMaxExperts; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  for (int r = 0; r < kFusedRounds; ++r) {
    const int64_t f = (int64_t)r * 1024 + tid;
    if (f < a.P) {
      bool valid;
      const int e = expert_of(a, f, valid);
      if (valid) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  const int n_e = tid < a.slots ? hist[tid] : 0;
  int total;
  const int off_e = block_exclusive_scan_1024(n_e, &total);
  if (tid < a.slots) {
    offsets[tid] = off_e;
    running[tid] = off_e;
    soff[tid] = off_e;
  }
  if (tid == 0) {
    offsets[a.slots] = total;
    soff[a.slots] = total;
  }

  const int lo[4] = {list_off.x, list_off.y, list_off.z, list_off.w};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int BM = kPlanBMs[b];
    const int tiles = tid < a.slots ? (n_e + BM - 1) / BM : 0;
    int ntiles;
    const int ts = block_exclusive_scan_1024(tiles, &ntiles);
    if (tid < a.slots) tstart[tid] = ts;
    if (tid == 0) {
      tstart[a.slots] = ntiles;
      plan[b] = ntiles;
      plan[4 + b] = lo[b];
    }
    __syncthreads();
    for (int slot = tid; slot < ntiles; slot += 1024) {
      int l = 0, h = a.slots;
      while (h - l > 1) {
        const int m = (l + h) >> 1;
        if (tstart[m] <= slot) l = m; else h = m;
      }
      write_tile(plan + lo[b] + 2 * slot, l, slot - tstart[l], BM, soff);
    }
    __syncthreads();
  }

  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kFusedRounds; ++r) {
    const int64_t f = (int64_t)r * 1024 + tid;
    const bool in = f < a.P;
    bool valid = false;
    const int e = in ? expert_of(a, f, valid) : 0;
    valid = valid && in;
    const int key = valid ? e : 2047;
    uint64_t same = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) {
      const bool bb = (key >> bit) & 1;
      const uint64_t bal = __ballot(bb);
      same &= bb ? bal : ~bal;
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

// ---------------------------------------------------------------- router
// One wavefront per token: k rounds of (max logit, lowest id) selection.
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
  __shared__ float sel_v[4][32];
  __shared__ int sel_i[4][32];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
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
      if (ok && (v[i] > bv || (v[i] == bv && lane + 64 * i < bi))) {
        bv = v[i];
        bi = lane + 64 * i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      sel_v[w][j] = bv;
      sel_i[w][j] = bi;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  if (lane < k) {
    const double top = (double)sel_v[w][0];
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += exp((double)sel_v[w][j] - top);
    const double mine = exp((double)sel_v[w][lane] - top);
    ids[(int64_t)t * k + lane] = sel_i[w][lane];
    wts[(int64_t)t * k + lane] = (float)(mine / sum);
  }
}

}  // namespace

AlignShape align_shape(int T, int topk, int E, int shared) {
  AlignShape a;
  a.T = T;
  a.topk = topk;
  a.E = E;
  a.shared = shared;
  a.P = (int64_t)T * topk + (int64_t)shared * T;
  a.slots = E + shared;
  a.nchunks = (int)((a.P + kAlignChunk - 1) / kAlignChunk);
  int64_t off = kPlanHeader;
  for (int b = 0; b < 4; ++b) {
    a.list_off[b] = off;
    a.list_len[b] = (a.P + kPlanBMs[b] - 1) / kPlanBMs[b] + a.slots;
    off += 2 * a.list_len[b];
  }
  return a;
}

size_t align_ws_bytes(const AlignShape& a) {
  return (size_t)a.nchunks * (size_t)a.slots * sizeof(int32_t);
}

size_t align_plan_ints(const AlignShape& a) { return (size_t)(a.list_off[3] + 2 * a.list_len[3]); }

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
  int4 lo0 = make_int4((int)a.list_off[0], (int)a.list_off[1], (int)a.list_off[2], (int)a.list_off[3]);
  if (a.P <= (int64_t)kFusedRounds * 1024) {
    align_fused_kernel<<<1, 1024, 0, s>>>(p, offsets, sorted_pair, inv_pos, plan, lo0);
    return hipGetLastError();
  }
  if (a.nchunks > 0) {
    align_count_kernel<<<a.nchunks, 256, 0, s>>>(p, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int4 lo = make_int4((int)a.list_off[0], (int)a.list_off[1], (int)a.list_off[2], (int)a.list_off[3]);
  align_scan_kernel<<<1, 1024, 0, s>>>(p, counts, offsets, plan, lo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nchunks == 0) return e;
  align_scatter_kernel<<<a.nchunks, 256, 0, s>>>(p, counts, sorted_pair, inv_pos);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  route_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace nvfp4
