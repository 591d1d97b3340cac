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

__device__ __forceinline__ float block_max(float m) {
  __shared__ float red[kThreads / kWave];
  // Reduce within the wave.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}

// One launch per call: grid (nblk, batches).  Every workgroup folds its
// maximum into ws_max[b] (float bits of a non-negative value order like
// unsigned integers), then counts itself in ws_cnt[b]; the last workgroup of a
// batch computes g[b] and puts both words back to zero, so the workspace is
// ready for the next call (it must be zero before the first one).
template <typename T>
__global__ __launch_bounds__(kThreads) void global_scale_kernel(const T* __restrict__ x, int64_t n,
                                                                float* __restrict__ g,
                                                                uint32_t* __restrict__ ws) {
  const int64_t b = blockIdx.y;
  const T* xb = x + b * n;
  const int64_t stride = (int64_t)gridDim.x * kThreads * 8;
  float m = 0.0f;
  for (int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8; i < n; i += stride) {
    float v[8];
    load8(xb, i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = block_max(m);
  if (threadIdx.x == 0) {
    uint32_t* ws_cnt = ws + 2 * b;
    uint32_t* ws_max = ws + 2 * b + 1;
    if (gridDim.x == 1) {
      g[b] = global_scale_of_amax(m);
      return;
    }
    __hip_atomic_fetch_max(ws_max, (uint32_t)__float_as_int(m), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t done = __hip_atomic_fetch_add(ws_cnt, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      const uint32_t bits = __hip_atomic_load(ws_max, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      g[b] = global_scale_of_amax(__int_as_float((int)bits));
      __hip_atomic_store(ws_max, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ws_cnt, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// One thread per 8 elements; the two threads of a 16-element block are
// adjacent lanes (K % 16 == 0 and the grid starts at an even index), so the
// block amax is one DPP exchange.  With x_deq, the exact f16 values of the
// codes (code * block scale, global scale not applied) are written as well:
// the grouped GEMMs read that copy instead of decoding the codes in every
// wavefront that uses them.
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const T* __restrict__ x, int64_t rows,
                                                            int64_t K, int64_t ldx,
                                                            const float* __restrict__ g,
                                                            int64_t rows_per_g,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            uint16_t* __restrict__ x_deq) {
  const int64_t hb_per_row = K >> 3;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * hb_per_row) return;  // whole lane pairs leave together
  const int64_t row = i / hb_per_row;
  quantize_half_block(x, row, (i - row * hb_per_row) << 3, K, ldx, g[row / rows_per_g], q, sf, x_deq);
}

int64_t amax_blocks(int64_t n) {
  // About 32 elements per thread; at most 1024 workgroups per batch.
  int64_t nb = (n + kThreads * 32 - 1) / (kThreads * 32);
  return nb < 1 ? 1 : (nb > 1024 ? 1024 : nb);
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
    global_scale_kernel<uint16_t><<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(x), n, g, w);
  else
    global_scale_kernel<float><<<grid, kThreads, 0, s>>>(static_cast<const float*>(x), n, g, w);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                           const float* g, int64_t rows_per_g, uint8_t* q, uint8_t* sf,
                           uint16_t* x_deq, hipStream_t s) {
  const int64_t threads = rows * (K >> 3);
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (dtype == 0)
    quantize_kernel<uint16_t><<<(unsigned)blocks, kThreads, 0, s>>>(
        static_cast<const uint16_t*>(x), rows, K, ldx, g, rows_per_g, q, sf, x_deq);
  else
    quantize_kernel<float><<<(unsigned)blocks, kThreads, 0, s>>>(
        static_cast<const float*>(x), rows, K, ldx, g, rows_per_g, q, sf, x_deq);
  return hipGetLastError();
}

}  // namespace nvfp4
