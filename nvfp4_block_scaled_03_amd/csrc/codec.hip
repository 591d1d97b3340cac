// NVFP4 global scale and block quantisation kernels (gfx950).
//
// Global scale g = fl32(amax / 2688) per tensor (activations) or per expert
// matrix (weights); block quantisation with one E4M3 scale per 16 elements
// and exact round-to-nearest-even decisions.  The per-block amax is taken in
// FP32 (FlashInfer #2723, "2. FP32 Amax Computation") with a wavefront (DPP)
// reduction across the two lanes that share a block.
#include "common.h"
#include "launch.h"
#include "quant.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kScaleThreads = 1024;  // global-scale workgroups

template <int NT>
__device__ __forceinline__ float block_max(float m) {
  __shared__ float red[NT / kWave];
  // Reduce within the wave.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}

// One launch per call: grid (nblk, batches).  Every workgroup folds its
// maximum into ws_max[b] (float bits of a non-negative value order like
// unsigned integers), then counts itself in ws_cnt[b]; the last workgroup of a
// batch computes g[b] and puts both words back to zero, so the workspace is
// ready for the next call (it must be zero before the first one).
//
// Each thread keeps U independent 16-byte loads in flight per trip; with the
// grid of amax_blocks a bf16 tensor is read in one trip, so the whole tensor
// is requested at once rather than in latency-bound rounds.
template <typename T>
__global__ __launch_bounds__(kScaleThreads) void global_scale_kernel(const T* __restrict__ x, int64_t n,
                                                                float* __restrict__ g,
                                                                uint32_t* __restrict__ ws) {
  constexpr int U = 8;
  constexpr int E = 16 / sizeof(T);  // elements per load
  const int64_t b = blockIdx.y;
  const T* xb = x + b * n;
  const int64_t stride = (int64_t)gridDim.x * kScaleThreads * E;
  float m = 0.0f;
  int64_t i = ((int64_t)blockIdx.x * kScaleThreads + threadIdx.x) * E;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    float v[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) load_vec(xb, i + u * stride, v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < E; ++j) m = fmaxf(m, amax_input(v[u][j]));
  }
  for (; i < n; i += stride) {
    float v[E];
    load_vec(xb, i, v);
#pragma unroll
    for (int j = 0; j < E; ++j) m = fmaxf(m, amax_input(v[j]));
  }
  m = block_max<kScaleThreads>(m);
  if (threadIdx.x == 0) {
    if (gridDim.x == 1) {
      g[b] = global_scale_of_amax(m);
      return;
    }
    fold_max_and_count(ws + 2 * b, ws + 2 * b + 1, m, gridDim.x, g + b);
  }
}

// One thread per 16-element block (BLOCK) or per 8 elements, the two
// threads of a block adjacent lanes that share its amax by one DPP exchange
// (K % 16 == 0 and the grid starts at an even index).  A lane per block takes
// the scale decision once per block; half a block per lane gives twice the
// lanes, which pays below about 2^18 blocks (the 512-expert layer's 65536
// blocks: 1 us faster; prefill's 524288: 2 us slower).  With x_deq, the exact
// f16 values of the codes (code * block scale, global scale not applied) are
// written as well: the grouped GEMMs read that copy instead of decoding the
// codes in every wavefront that uses them.
constexpr int64_t kBlockLaneMin = int64_t(1) << 18;   // blocks from which a lane takes a whole block

template <typename T, bool BLOCK>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const T* __restrict__ x, int64_t rows,
                                                            int64_t K, int64_t ldx,
                                                            const float* __restrict__ g,
                                                            int64_t rows_per_g,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            uint16_t* __restrict__ x_deq) {
  const int64_t per_row = K >> (BLOCK ? 4 : 3);
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * per_row) return;  // (half blocks: whole lane pairs leave together)
  const int64_t row = i / per_row;
  const int64_t c = (i - row * per_row) << (BLOCK ? 4 : 3);
  if constexpr (BLOCK) {
    quantize_block(x, row, c, K, ldx, g[row / rows_per_g], q, sf, x_deq);
  } else {
    float v[8];
    load8(x, row * ldx + c, v);
    quantize_half_block_values(v, row, c, K, g[row / rows_per_g], q, sf, x_deq);
  }
}

int64_t amax_blocks(int64_t n) {
  // 64 elements per thread (one trip of 8 loads for bf16), at most 128
  // workgroups per batch: the workgroups meet in two atomics on one address
  // each, and those serialise (measured on a 16.7 MB tensor: 512 workgroups
  // 17 us, 256 of a quarter the threads 11.5 us).
  int64_t nb = (n + kScaleThreads * 64 - 1) / (kScaleThreads * 64);
  return nb < 1 ? 1 : (nb > 128 ? 128 : nb);
}

}  // namespace

size_t global_scale_ws_bytes(int64_t batches, int64_t n) {
  (void)n;
  return (size_t)batches * 2 * sizeof(uint32_t);
}

hipError_t launch_global_scale(const void* x, int dtype, int64_t batches, int64_t n, float* g,
                               void* ws, hipStream_t s) {
  const int64_t nb = amax_blocks(n);
  dim3 grid((unsigned)nb, (unsigned)batches);
  uint32_t* w = static_cast<uint32_t*>(ws);
  if (dtype == 0)
    global_scale_kernel<uint16_t><<<grid, kScaleThreads, 0, s>>>(static_cast<const uint16_t*>(x), n, g, w);
  else
    global_scale_kernel<float><<<grid, kScaleThreads, 0, s>>>(static_cast<const float*>(x), n, g, w);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                           const float* g, int64_t rows_per_g, uint8_t* q, uint8_t* sf,
                           uint16_t* x_deq, hipStream_t s) {
  const bool block = rows * (K >> 4) >= kBlockLaneMin;
  const int64_t threads = rows * (K >> (block ? 4 : 3));
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const float* xf = static_cast<const float*>(x);
  if (dtype == 0 && block)
    quantize_kernel<uint16_t, true><<<(unsigned)blocks, kThreads, 0, s>>>(xb, rows, K, ldx, g, rows_per_g, q, sf, x_deq);
  else if (dtype == 0)
    quantize_kernel<uint16_t, false><<<(unsigned)blocks, kThreads, 0, s>>>(xb, rows, K, ldx, g, rows_per_g, q, sf, x_deq);
  else if (block)
    quantize_kernel<float, true><<<(unsigned)blocks, kThreads, 0, s>>>(xf, rows, K, ldx, g, rows_per_g, q, sf, x_deq);
  else
    quantize_kernel<float, false><<<(unsigned)blocks, kThreads, 0, s>>>(xf, rows, K, ldx, g, rows_per_g, q, sf, x_deq);
  return hipGetLastError();
}

}  // namespace nvfp4
