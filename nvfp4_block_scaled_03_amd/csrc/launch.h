// Internal launch functions behind the C ABI (host side).  Arguments are
// validated by api.hip before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// Tile lists of the alignment plan, in this order: lists 0-3 cover every
// expert with tiles of 16, 32, 64 and 128 rows; list 4 covers only the
// experts with at most kSplitRows rows (16-row tiles) and list 5 only those
// with more (128-row tiles), so that a batch whose experts differ widely in
// rows can run its short experts on the streaming kernel and its tall ones
// on the 128-row kernel.  Plan layout (int32): counts[6], list offsets[6],
// then per list 2 ints per tile {expert | m_tile << 11, first row | rows << 24},
// expert-major.
constexpr int kPlanLists = 6;
constexpr int kPlanBMs[kPlanLists] = {16, 32, 64, 128, 16, 128};
constexpr int kSplitRows = 32;
constexpr int kPlanHeader = 2 * kPlanLists;
struct PlanOffs {
  int v[kPlanLists];
};
// Whether list b holds the tiles of an expert with n rows.
__host__ __device__ constexpr bool plan_list_has(int b, int n) {
  return b < 4 ? true : (b == 4 ? n <= kSplitRows : n > kSplitRows);
}
constexpr int kMaxExperts = 1024;

size_t global_scale_ws_bytes(int64_t batches, int64_t n);
hipError_t launch_global_scale(const void* x, int dtype, int64_t batches, int64_t n, float* g,
                               void* ws, hipStream_t s);
hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                           const float* g, int64_t rows_per_g, uint8_t* q, uint8_t* sf,
                           uint16_t* x_deq, hipStream_t s);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);

struct AlignShape {
  int T, topk, E, shared, H;
  int64_t P;        // pairs
  int slots;        // E + shared
  int nchunks;      // pair chunks of kAlignChunk
  int64_t list_off[kPlanLists];
  int64_t list_len[kPlanLists];
};
constexpr int kAlignChunk = 1024;
AlignShape align_shape(int T, int topk, int E, int shared);
size_t align_ws_bytes(const AlignShape& a);
size_t align_plan_ints(const AlignShape& a);
hipError_t launch_align(const AlignShape& a, const int32_t* topk_ids, int32_t* offsets,
                        int32_t* sorted_pair, int32_t* inv_pos, int32_t* plan, void* ws,
                        hipStream_t s);
// Activation global scale (bf16 x [T][H]) and alignment in one launch when
// the pairs fit one workgroup, else the two launches in sequence.
// OCP MXFP4 quantisation of bf16 x [T][H] (canonical q, ex) and the
// alignment: one launch when the pairs fit one workgroup, else the count and
// scan launches then the scatter beside the quantisation.
hipError_t launch_mx_quantize_and_align(const AlignShape& a, const uint16_t* x, uint8_t* q, uint8_t* ex,
                                       const int32_t* topk_ids, int32_t* offsets, int32_t* sorted_pair,
                                       int32_t* inv_pos, int32_t* plan, void* ws, hipStream_t s);
hipError_t launch_scale_and_align(const AlignShape& a, const uint16_t* x, float* g, void* gs_ws,
                                  const int32_t* topk_ids, int32_t* offsets, int32_t* sorted_pair,
                                  int32_t* inv_pos, int32_t* plan, void* ws, hipStream_t s);
// Global scale, NVFP4 quantisation (+ optional exact f16 copy) and alignment:
// one launch when the activations are decode-sized (T * H <= 2^18 and the
// pairs fit one workgroup), else scale_and_align followed by quantize.
// Router then alignment (two launches).
hipError_t launch_route_and_align(const AlignShape& a, const float* logits, int32_t* ids, float* w,
                                  int32_t* offsets, int32_t* sorted_pair, int32_t* inv_pos,
                                  int32_t* plan, void* ws, hipStream_t s);
hipError_t launch_quantize_and_align(const AlignShape& a, const uint16_t* x, float* g, void* gs_ws,
                                    uint8_t* q, uint8_t* sf, uint16_t* x_deq,
                                    const int32_t* topk_ids, int32_t* offsets, int32_t* sorted_pair,
                                    int32_t* inv_pos, int32_t* plan, void* ws, hipStream_t s);

// Weight streaming layout.  For an expert matrix [N][K] (N output columns,
// K contraction, KC = K/128 chunks): codes [N/16][KC][64 lanes][16 B]
// followed (after all experts' codes) by scales
// [N/32][KC/G][64 lanes][G chunks][2 tiles][2 B], G = scale_group(KC): a
// lane's scale bytes of G consecutive chunks are contiguous (one load).
__host__ __device__ constexpr int scale_group(int kc) {
  return kc % 4 == 0 ? 4 : kc % 3 == 0 ? 3 : kc % 2 == 0 ? 2 : 1;
}
// Byte offset, inside one expert's scale block, of the 4-byte word of column
// tile pair tp, chunk kc, lane (the word holds 2 tiles x 2 scale bytes).
__host__ __device__ constexpr int64_t scale_word_offset(int64_t tp, int kc, int KC, int lane) {
  const int G = scale_group(KC);
  return ((tp * (KC / G) + kc / G) * 64 + lane) * (4 * G) + (kc % G) * 4;
}
size_t prep_bytes(int64_t slots, int64_t N, int64_t K);
hipError_t launch_prep(int64_t slots, int64_t N, int64_t K, int interleave_I, const uint8_t* q,
                       const uint8_t* sf, uint8_t* prep, hipStream_t s);

struct GemmArgs {
  // dims
  int T, topk, E, shared, H, I;
  int64_t P;
  // routing
  const int32_t* offsets;
  const int32_t* sorted_pair;  // GEMM1 only
  const int32_t* inv_pos;      // combine only
  const int32_t* plan;
  const float* topk_w;
  // operands
  const uint8_t* a_q;
  const uint8_t* a_sf;
  const uint16_t* a_h;  // bf16 activations (W4A16) or the f16 dequantised copy (W4A4, optional)
  const float* g_a;     // activation global scale (W4A4) or null
  const uint8_t* w_prep;
  const float* g_w;
  // GEMM1 outputs
  const float* g2;
  uint8_t* out_q;
  uint8_t* out_sf;
  uint16_t* out_h;      // bf16 intermediate (W4A16) or its optional f16 copy (W4A4)
  // GEMM2 outputs
  float* d_ws;
  void* out;
  int out_dtype;
  // Which share of the work a call launches (kPart*): all of it, the
  // short-expert list or the tall-expert list of a split layer, or the
  // combine alone.
  int part;
};
constexpr int kPartAll = 0, kPartShort = 1, kPartTall = 2, kPartCombine = 3;
hipError_t launch_gemm1(const GemmArgs& a, bool w4a4, hipStream_t s);
// Whether the W4A4 GEMMs run faster on the exact f16 activation copies than
// on the codes for these dimensions (the wide 128-row-tile kernel).
bool prefers_decoded(int T, int topk, int E, int shared);
hipError_t launch_gemm2_combine(const GemmArgs& a, bool w4a4, hipStream_t s);
// out[t] = sum_j topk_w[t][j] * d[inv_pos[t*topk + j]] (+ the shared row),
// FP32 in j order, rows with inv_pos < 0 skipped; out bf16 (0) or f32 (1).
hipError_t launch_combine(const float* d, const int32_t* inv_pos, const float* topk_w, int T, int topk,
                          int shared, int H, void* out, int out_dtype, hipStream_t s);
// Tile list (0..3: 16, 32, 64, 128 rows) chosen from the mean rows per expert.
int pick_list(int64_t P, int slots);
// Whether short experts and tall ones run on different kernels (lists 4 and
// 5): short tiles on average (the streaming regime) while one expert may
// still hold more than 64 rows (T > 64, or a shared expert, which takes
// every token).
bool split_experts(const AlignShape& al);

// Dense linear y [M][N] = x [M][K] W^T on the grouped-GEMM kernels with one
// expert (plan from an alignment of M pairs to expert 0).
struct LinearArgs {
  int64_t M, N, K;
  bool w4a4;
  const int32_t* plan;
  const uint8_t* w_prep;   // streaming layout of W [N][K] (one expert)
  const float* g_w;        // weight global scale
  const float* g_a;        // activation global scale (W4A4) or null
  const uint8_t* a_q;      // W4A4 codes [M][K/2] + scales, or
  const uint8_t* a_sf;
  const uint16_t* a_h;     // the exact f16 copy (W4A4) / bf16 x (W4A16)
  void* out;
  int out_dtype;           // 0 bf16, 1 f32
};
hipError_t launch_linear(const LinearArgs& a, hipStream_t s);

}  // namespace nvfp4
