// Host entry points of the OCP MXFP4 kernels (mx.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// OCP MXFP4 (E8M0 scale per 32): quantisation (dtype 0 bf16, 1 f32; codes
// [rows][K/2], scale bytes [rows][K/32]), weight prep and the dense GEMM on
// the scaled FP4 matrix instruction (out_dtype 0 bf16, 1 f32).
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, uint8_t* q,
                              uint8_t* ex, hipStream_t s);
// The GEMM's activation operand: x bf16 [M][K] quantised into the operand
// layout (rows padded with zeros to mx_rows_pad(M); codes mx_rows_pad(M) K/2
// bytes, scales mx_rows_pad(M) K/32 bytes; K % 128 == 0).
int64_t mx_rows_pad(int64_t M);
hipError_t launch_mx_quantize_operand(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* ex,
                                      hipStream_t s);
size_t mx_prep_bytes(int64_t N, int64_t K);
hipError_t launch_mx_prep(int64_t N, int64_t K, const uint8_t* q, const uint8_t* ex, uint8_t* prep,
                          hipStream_t s);
// a_q / a_e: the activation operand from launch_mx_quantize_operand.
hipError_t launch_mx_gemm(const uint8_t* a_q, const uint8_t* a_e, int64_t M, int64_t N, int64_t K,
                          const uint8_t* w_prep, void* out, int out_dtype, hipStream_t s);

// Mixture-of-experts layer in MXFP4: expert weights prepared per slot
// (interleave_I = I for the gate/up weights: column tiles alternate gate and
// up), GEMM1 with SwiGLU and MXFP4 requantisation of h, GEMM2 into the FP32
// per-row workspace followed by the combine.  Activations in the canonical
// MXFP4 layout (codes [rows][K/2], exponent bytes [rows][K/32]).
size_t mx_expert_prep_bytes(int64_t slots, int64_t N, int64_t K);
hipError_t launch_mx_expert_prep(int64_t slots, int64_t N, int64_t K, int interleave_I, const uint8_t* q,
                                 const uint8_t* ex, uint8_t* prep, hipStream_t s);
struct MxGemmArgs {
  int T, topk, E, shared, H, I;
  const int32_t* sorted_pair;   // GEMM1
  const int32_t* inv_pos;       // combine
  const int32_t* plan;
  const float* topk_w;
  const uint8_t* a_q;           // a1 (GEMM1) or a2 (GEMM2) codes
  const uint8_t* a_e;           // and exponent bytes
  const uint8_t* w_prep;
  uint8_t* out_q;               // GEMM1: a2
  uint8_t* out_e;
  float* d_ws;                  // GEMM2: FP32 [P][H]
  void* out;
  int out_dtype;
  int part;                     // share of the work, as GemmArgs::part
};
hipError_t launch_mx_gemm1_swiglu(const MxGemmArgs& a, hipStream_t s);
hipError_t launch_mx_gemm2_combine(const MxGemmArgs& a, hipStream_t s);

}  // namespace nvfp4
