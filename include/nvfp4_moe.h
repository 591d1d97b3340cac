/*
 * nvfp4_moe.h -- C ABI of libnvfp4moe.so, the NVFP4 mixture-of-experts expert
 * path for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title -> short tag):
 *   "[Kernel] Add NVFP4 MoE CUTLASS support for SM120"               vLLM PR #29242
 *   "SM120 (RTX Blackwell) NVFP4 MoE: CUTLASS Grouped Block-Scaled
 *    GEMM Produces Invalid Output; FlashInfer Requires Extensive
 *    Patching"                                                      FlashInfer #2723
 *   "[NVFP4] NVFP4 MOE emulation fallback for H100/MI300/MI350, ..." vLLM PR #35737
 *   "Report: NVFP4 kernel selection on SM120/SM121"                 unsloth PR #10417
 *
 * The path (one layer):
 *   nvfp4_global_scale  activations -> g1                    (W4A4 only)
 *   nvfp4_quantize      activations, g1 -> a1 codes + scales (W4A4 only)
 *   moe_align           top-k expert ids -> rows grouped by expert
 *   (moe_scale_and_align: the first and third steps in one call;
 *    moe_quantize_and_align: the first three)
 *   grouped_gemm1_swiglu[_w4a16]   gate/up GEMM, SwiGLU, requantisation
 *   grouped_gemm2_combine[_w4a16]  down GEMM, top-k weighted combine
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless stated; `dims` is a host pointer.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL is the null stream).  The library never synchronises, never
 *   allocates or frees device memory, and keeps no state between calls: all
 *   scratch memory is a caller-owned workspace sized by the *_size queries.
 *   (One exception, for callers that cannot allocate:
 *   grouped_gemm2_combine_noalloc keeps its scratch in a static device array
 *   per GPU; see its declaration.)  Calls that touch the same buffers must be
 *   ordered by the caller.
 * - The caller owns every buffer.  Nothing is retained after a call returns.
 * - bfloat16 buffers are passed as uint16_t*.
 * - Canonical NVFP4 layout (the layout bit-exactness is judged on): a matrix
 *   [rows][K] is stored as codes uint8 [rows][K/2] -- element 2j in the low
 *   nibble of byte j, element 2j+1 in the high nibble, each a 4-bit E2M1 code
 *   (sign | 2 exponent bits | 1 mantissa bit, bias 1) -- and scales uint8
 *   [rows][K/16], one unsigned E4M3 (OCP "FN", bias 7) byte per 16
 *   consecutive elements.  A value is E2M1[code] * E4M3[scale] * g with one
 *   FP32 global scale g per tensor (activations) or per expert matrix
 *   (weights).  The element type and the per-16 unsigned E4M3 scale are those
 *   of the native block-scaled instruction named in unsloth PR #10417 ("Why it
 *   matters"); "FP4 weights with FP8 block scales" is FlashInfer #2723
 *   ("Model" table).
 * - Errors: every argument is validated on the host before anything is
 *   launched.  A failing call returns a negative NVFP4_E* code, launches
 *   nothing, writes nothing, and sets a thread-local message readable with
 *   nvfp4_last_error(); GEMM messages carry num_experts, M, N, K and the
 *   workspace size, like the grouped-GEMM initialisation error in vLLM PR
 *   #29242 (review of nvfp4_blockwise_moe_kernel.cu).  A failed kernel launch
 *   returns NVFP4_ELAUNCH with the HIP error string.  Values that live on the
 *   device (expert ids, per-expert row counts) cannot be checked on the host:
 *   out-of-range expert ids are dropped (see moe_align), and row counts come
 *   from moe_align and are trusted, as the per-group shapes of the grouped
 *   GEMM in vLLM PR #29242 (debug trace) are device-resident and unchecked.
 * - Inputs must be finite; NaN or Inf inputs give unspecified (but in-bounds)
 *   results, with one guarantee: a NaN takes no part in any maximum (the
 *   global and the per-block amax ignore it), on every dispatch path, so the
 *   fused and unfused activation paths agree bit for bit on every input.
 * - T == 0: the layer calls (moe_*, grouped_gemm*) check dims and return
 *   NVFP4_OK without launching or writing anything; their pointers may then
 *   be NULL.  rows == 0 / M == 0 is the same no-op for the row-wise calls.
 */
#ifndef NVFP4_MOE_H
#define NVFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_MOE_ABI_VERSION 9

/* Status codes. */
#define NVFP4_OK 0
#define NVFP4_EINVAL (-1)     /* null pointer, bad enum, misaligned pointer   */
#define NVFP4_ESHAPE (-2)     /* unsupported or inconsistent dimensions       */
#define NVFP4_EWORKSPACE (-3) /* workspace smaller than the size query        */
#define NVFP4_ELAUNCH (-4)    /* a kernel launch failed (HIP error in message) */

/* Element types of dense inputs/outputs. */
#define NVFP4_BF16 0
#define NVFP4_F32 1

/* Layer dimensions (host struct).
 *   T      tokens (>= 0)
 *   topk   routed experts per token (1..E)
 *   E      routed experts (>= 1)
 *   H      hidden size; multiple of 128 (contraction of GEMM1, output of GEMM2)
 *   I      expert intermediate size; multiple of 128
 *   shared 0 or 1; 1 adds an always-on shared expert as expert slot E, which
 *          every token visits with weight 1 (the "512 routed + 1 shared"
 *          layout of FlashInfer #2723, "Model" table)
 * E + shared <= 1024.  P = T*topk + shared*T is the number of (token, expert)
 * pairs, i.e. of rows in the grouped GEMMs; P < 2^31. */
typedef struct nvfp4_moe_dims {
  int32_t T;
  int32_t topk;
  int32_t E;
  int32_t H;
  int32_t I;
  int32_t shared;
} nvfp4_moe_dims;

/* ABI version of the loaded library (NVFP4_MOE_ABI_VERSION). */
int nvfp4_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  The pointer is
 * valid until the next library call on the same thread. */
const char* nvfp4_last_error(void);

/* ------------------------------------------------------------------------ */
/* Global scale.                                                             */
/* ------------------------------------------------------------------------ */
/* g[b] = fl32(max_i |x[b][i]| / 2688) for b < batches, over n contiguous
 * elements per batch (x is [batches][n], dtype NVFP4_BF16 or NVFP4_F32).
 * 2688 = 6 * 448, the largest E2M1 magnitude times the largest E4M3 scale, so
 * the block holding the tensor's amax gets the top E4M3 scale.  The pages fix
 * FP32 for the scale arithmetic (FlashInfer #2723, "2. FP32 Amax
 * Computation"); the amax itself is exact.  The quotient is correctly rounded.
 * Use batches = 1 for an activation tensor, batches = experts for a stack of
 * expert weight matrices.
 * ws: workspace of nvfp4_global_scale_workspace_size(batches, n) bytes (8
 * per batch), 4-byte aligned, which must be zero-filled before its first use:
 * the call folds partial maxima into it across workgroups and leaves it zero
 * again when it finishes, so one buffer serves every later call on the same
 * stream (concurrent calls need separate buffers).  x must be 16-byte aligned
 * and n a multiple of 8. */
size_t nvfp4_global_scale_workspace_size(int64_t batches, int64_t n);
int nvfp4_global_scale(const void* x, int dtype, int64_t batches, int64_t n, float* g,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Quantisation to NVFP4.                                                    */
/* ------------------------------------------------------------------------ */
/* Encode rows of x ([rows][ldx] elements, dtype NVFP4_BF16 or NVFP4_F32, the
 * first K of each row used) into canonical NVFP4: q uint8 [rows][K/2], sf
 * uint8 [rows][K/16].  Row r uses the global scale g[r / rows_per_g] (a device
 * array): rows_per_g = rows for one activation tensor, rows_per_g = N for a
 * stack of [N][K] expert matrices.
 * Per 16-element block: s = round(amax / (6 g)) to the nearest E4M3 value,
 * ties to the even code, saturating at 448; each element gets sign(x) |
 * round(|x| / (s g)) to the nearest E2M1 magnitude, ties to even, saturating
 * at 6; a block with s = 0 gets magnitude 0 everywhere.  Decisions are exact
 * (taken on the real quotients).  This is the per-token activation
 * quantisation of FlashInfer #2723 ("Why 39 vs 49 tok/s?"), with per-block
 * amax by a wavefront reduction in FP32 ("2. FP32 Amax Computation").
 * x_deq (optional, may be NULL): IEEE half [rows][K] receiving the exact
 * value E2M1[code] * E4M3[scale] of every element (the global scale is not
 * applied; six significant bits at most and |value| <= 2688, so the half is
 * exact).  The grouped GEMMs accept this copy in place of the codes: on
 * gfx950 the FP4 conversion instructions run at a quarter of the VALU rate,
 * and decoding each activation once here saves decoding it in every
 * wavefront that reads it.
 * Requirements: K % 16 == 0, ldx >= K, ldx % 8 == 0, x and x_deq 16-byte
 * aligned, q 4-byte aligned, g != NULL, rows_per_g >= 1. */
int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                   const float* g, int64_t rows_per_g, uint8_t* q, uint8_t* sf, uint16_t* x_deq,
                   void* stream);

/* ------------------------------------------------------------------------ */
/* Router (runs before the path; not part of the timed layer).               */
/* ------------------------------------------------------------------------ */
/* Softmax / top-k / renormalise router over FP32 logits [T][E]: ids int32
 * [T][topk] are the topk largest logits in decreasing order (equal logits:
 * lower id first) and weights float32 [T][topk] the softmax over the selected
 * logits (equal to the full softmax renormalised over the selection).  The
 * pages route each token to its top experts ("10 routed per token",
 * FlashInfer #2723, "Model" table) without spelling out the router; this is
 * the usual reading.  1 <= topk <= min(E, 32), E <= 1024. */
int moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t topk, int32_t* ids,
                   float* weights, void* stream);

/* Router and permutation in one call: the same results, bit for bit, as
 * moe_route_topk(logits, T, E, topk, topk_ids, topk_w) followed by
 * moe_align(dims, topk_ids, ...), with moe_align's dims, output and
 * workspace contracts (topk <= 32 for the router).  logits float32 [T][E];
 * topk_ids int32 [T][topk] and topk_w float32 [T][topk] are written.  The
 * two steps run as two launches on the stream (the router is a per-token
 * latency chain; one workgroup doing both measured slower). */
int moe_route_and_align(const nvfp4_moe_dims* dims, const float* logits, int32_t* topk_ids,
                        float* topk_w, int32_t* expert_offsets, int32_t* sorted_pair, int32_t* inv_pos,
                        int32_t* plan, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Permutation by expert.                                                    */
/* ------------------------------------------------------------------------ */
/* Group the P (token, expert) pairs by expert, the role of
 * get_cutlass_moe_mm_data in vLLM PR #29242 (commit list).  Pair f = t*topk+j
 * has expert topk_ids[t][j]; with dims->shared, pair T*topk + t has expert E.
 * Outputs (all exact integers):
 *   expert_offsets int32 [E+shared+1]: rows of expert e are
 *                  offsets[e] <= p < offsets[e+1]; offsets[E+shared] = number
 *                  of kept pairs.
 *   sorted_pair    int32 [P]: the pair index f at row p; within an expert,
 *                  rows are in increasing f (a stable sort by expert).
 *   inv_pos        int32 [P]: row of pair f, or -1 when its expert id is
 *                  outside [0, E) (such pairs are dropped and contribute
 *                  nothing).
 *   plan           int32 [moe_align_plan_size/4]: opaque tile lists consumed
 *                  by the grouped GEMMs (must come from a moe_align call with
 *                  the same dims).
 * ws: moe_align_workspace_size(dims) bytes of scratch. */
size_t moe_align_workspace_size(const nvfp4_moe_dims* dims);
size_t moe_align_plan_size(const nvfp4_moe_dims* dims);
int moe_align(const nvfp4_moe_dims* dims, const int32_t* topk_ids, int32_t* expert_offsets,
              int32_t* sorted_pair, int32_t* inv_pos, int32_t* plan, void* ws, size_t ws_bytes,
              void* stream);

/* The activation global scale and the permutation in one call: the same
 * results as nvfp4_global_scale(x, NVFP4_BF16, 1, T*H, g1, gs_ws, ...)
 * followed by moe_align(dims, topk_ids, ...), with the same workspace
 * contracts.  The two steps are independent, so when the pairs fit one
 * workgroup (P <= 4096) they share one kernel launch; otherwise they run as
 * the two launches.  x is bfloat16 [T][H], 16-byte aligned. */
int moe_scale_and_align(const nvfp4_moe_dims* dims, const uint16_t* x, float* g1, void* gs_ws,
                        size_t gs_ws_bytes, const int32_t* topk_ids, int32_t* expert_offsets,
                        int32_t* sorted_pair, int32_t* inv_pos, int32_t* plan, void* ws,
                        size_t ws_bytes, void* stream);

/* Global scale, quantisation and permutation in one call: the same results,
 * bit for bit, as moe_scale_and_align(dims, x, g1, gs_ws, ...) followed by
 * nvfp4_quantize(x, NVFP4_BF16, T, H, H, g1, T, a1_q, a1_sf, a1_deq, ...),
 * with the same argument contracts (a1_q [T][H/2] 4-byte aligned, a1_sf
 * [T][H/16], a1_deq optional f16 [T][H] 16-byte aligned).  The three steps of
 * FlashInfer #2723's activation path ("2. FP32 Amax Computation", the
 * per-token quantisation of "Why 39 vs 49 tok/s?") and the permutation of
 * vLLM PR #29242 (get_cutlass_moe_mm_data) need no ordering among
 * themselves beyond g1 before the codes; for decode-sized activations
 * (T*H <= 2^18, P <= 4096) they run as one launch in which every quantising
 * workgroup computes the exact amax itself; beyond that (P > 4096 or
 * T*H > 2^18) as three launches (per-workgroup maxima of |x| beside the
 * expert counts; the scan, which also reduces the maxima to g1; the pair
 * scatter and tile lists beside the quantisation), which keep their partial
 * maxima in ws and leave gs_ws untouched; dense use (no ids, one expert, P
 * <= 4096) as moe_scale_and_align then nvfp4_quantize.  Errors as for those
 * calls. */
int moe_quantize_and_align(const nvfp4_moe_dims* dims, const uint16_t* x, float* g1, void* gs_ws,
                           size_t gs_ws_bytes, uint8_t* a1_q, uint8_t* a1_sf, uint16_t* a1_deq,
                           const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pair,
                           int32_t* inv_pos, int32_t* plan, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Dense NVFP4 linear layer (the same kernels with one expert).              */
/* ------------------------------------------------------------------------ */
/* y [M][N] = x [M][K] W^T for an NVFP4 weight W [N][K] with global scale gw,
 * the per-GEMM workload the pages time across batch sizes M with NVFP4
 * activations against bf16 activations and weight dequantisation (unsloth
 * PR #10417, "Why it matters").  x is bfloat16 [M][K] (16-byte aligned); the
 * weight is prepared by nvfp4_prep_weights(dims, 2, ...) with dims
 * {T: any, topk: 1, num_experts: 1, H: N, I: K, shared: 0} (the down
 * projection's layout of one expert).  N and K are multiples of 128.
 *   nvfp4_linear:        W4A4.  x gets a dynamic global scale and NVFP4
 *                        quantisation (as nvfp4_global_scale + nvfp4_quantize),
 *                        then y = g * gw * (x_hat W_hat^T) with FP32
 *                        accumulation.
 *   nvfp4_linear_w4a16:  W4A16.  y = gw * (x W_hat^T).
 * out: bfloat16 (out_dtype 0, round to nearest even) or float32 (1) [M][N].
 * ws: nvfp4_linear_workspace_size(M, N, K, w4a4) bytes, 256-byte aligned,
 * zero-filled before its first use (the library leaves its counter words
 * zero after every call).  Errors: NVFP4_ESHAPE, NVFP4_EINVAL,
 * NVFP4_EWORKSPACE (message names M, N, K and the sizes). */
size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int w4a4);
int nvfp4_linear(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_prep,
                 const float* gw, void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream);
int nvfp4_linear_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_prep,
                       const float* gw, void* out, int out_dtype, void* ws, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Dense OCP MXFP4 linear layer on the scaled FP4 matrix instruction.        */
/* ------------------------------------------------------------------------ */
/* The emulation backend's other block format, OCP MXFP4 on MI3xx (vLLM PR
 * #35737, summary), built natively: CDNA4's scaled FP4 matrix instruction
 * takes E2M1 codes with one E8M0 scale per 32 elements of each operand row,
 * so the codes are multiplied as stored, with no decoding step.
 * Canonical MXFP4 layout: codes uint8 [rows][K/2] packed as for NVFP4 and
 * exponent bytes uint8 [rows][K/32] (E8M0: the scale is 2^(byte - 127)).
 * Quantisation of a block of 32 with largest magnitude amax: byte =
 * clamp(floor(log2 amax) - 2 + 127, 0, 254), 0 for a block of zeros; each
 * element is v / 2^(byte - 127) rounded to the nearest E2M1 value (ties to
 * the even code, above 6 saturating to 6), its sign kept.  No global scale.
 *
 * mxfp4_quantize: x [rows][ldx] (dtype 0 bfloat16, 1 float32; 16-byte
 *   aligned, ldx a multiple of 8, K a multiple of 32, rows * K < 2^31) ->
 *   q [rows][K/2] (4-byte aligned), ex [rows][K/32].  Bit-exact.
 * mxfp4_prep_weights: canonical weight W [N][K] (q 16-byte aligned) -> prep
 *   (mxfp4_prep_weights_size bytes, 16-byte aligned; the same bytes
 *   permuted).  N, K multiples of 128.
 * mxfp4_linear: y [M][N] = x_hat W_hat^T with FP32 accumulation, x bfloat16
 *   [M][K] (16-byte aligned, M K < 2^31, the prepared weight below 4 GiB)
 *   quantised on the fly into the workspace (ws:
 *   mxfp4_linear_workspace_size bytes, 256-byte aligned, no initial
 *   contents needed).  out as nvfp4_linear.  Errors: NVFP4_ESHAPE,
 *   NVFP4_EINVAL, NVFP4_EWORKSPACE. */
int mxfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, uint8_t* q,
                   uint8_t* ex, void* stream);
size_t mxfp4_prep_weights_size(int64_t N, int64_t K);
int mxfp4_prep_weights(int64_t N, int64_t K, const uint8_t* q, const uint8_t* ex, uint8_t* prep,
                       void* stream);
size_t mxfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K);
int mxfp4_linear(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_prep, void* out,
                 int out_dtype, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Weight preparation (offline).                                             */
/* ------------------------------------------------------------------------ */
/* Rearrange canonical NVFP4 expert weights into the library's streaming
 * layout `prep` (opaque; the same bytes, permuted).  which = 13: the gate/up
 * weights q [E+shared][2I][H/2], sf [E+shared][2I][H/16] (rows [0, I) gate,
 * rows [I, 2I) up); which = 2: the down weights q [E+shared][H][I/2], sf
 * [E+shared][H][I/16].  prep must hold nvfp4_prep_weights_size bytes and be
 * 16-byte aligned. */
size_t nvfp4_prep_weights_size(const nvfp4_moe_dims* dims, int which);
int nvfp4_prep_weights(const nvfp4_moe_dims* dims, int which, const uint8_t* q, const uint8_t* sf,
                       uint8_t* prep, void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped expert GEMMs.                                                     */
/* ------------------------------------------------------------------------ */
/* GEMM1 (W4A4).  For every row p of expert e (token t = the token of pair
 * sorted_pair[p]):
 *   c = alpha1[e] * (a1_hat[t] . w13_hat[e]^T)      (FP32 accumulation)
 *   h = silu(c[0:I]) * c[I:2I]                      silu(z) = z / (1 + e^-z)
 *   a2 row p = NVFP4 encoding of h with global scale *g2 (as nvfp4_quantize)
 * where a1_hat, w13_hat are the dequantised codes times block scales and
 * alpha1[e] = fl32((*g1) * gw13[e]): the per-expert FP32 alpha with no C input
 * of the grouped GEMM epilogue in vLLM PR #29242 (review of
 * nvfp4_blockwise_moe_kernel.cu).  g1 is a device scalar (nvfp4_global_scale
 * output), gw13 a device array [E+shared], g2 a device scalar chosen by the
 * caller (a static calibration of the intermediate).  Outputs a2_q uint8
 * [P][I/2] and a2_sf uint8 [P][I/16] are in sorted-row order.  a1_q/a1_sf are
 * the canonical [T][H/2] / [T][H/16] activations.
 * a1_deq (optional): the x_deq output of nvfp4_quantize for a1_q/a1_sf, half
 * [T][H]; when given, it is read instead of the codes (which may then be
 * NULL) -- the same values, decoded once.  a2_deq (optional output): half
 * [P][I], the exact values of the a2 codes (as x_deq), for GEMM2. */
int grouped_gemm1_swiglu(const nvfp4_moe_dims* dims, const uint8_t* a1_q, const uint8_t* a1_sf,
                         const uint16_t* a1_deq, const float* g1, const int32_t* sorted_pair,
                         const int32_t* expert_offsets, const int32_t* plan,
                         const uint8_t* w13_prep, const float* gw13, const float* g2,
                         uint8_t* a2_q, uint8_t* a2_sf, uint16_t* a2_deq, void* stream);

/* 1 when, for these dimensions, the W4A4 GEMMs are faster given the exact
 * f16 activation copies (a1_deq from nvfp4_quantize, a2_deq from GEMM1) than
 * given the codes alone, else 0 (also 0 for invalid dims): tall tiles on
 * average, or short ones on average while some expert may still exceed 64
 * rows (T > 64 or a shared expert) -- then, given the copies, the GEMMs run
 * the experts with more than 32 rows on the 128-row kernel and the rest on
 * the streaming kernel.  A performance hint only: both inputs give the same
 * results. */
int grouped_gemm_prefers_decoded(const nvfp4_moe_dims* dims);

/* Workspace of the GEMM2 calls: the per-row FP32 down-projection outputs
 * [P][H] that the combine reads. */
size_t grouped_gemm_workspace_size(const nvfp4_moe_dims* dims);

/* GEMM2 (W4A4) + combine.  For every row p of expert e:
 *   d[p] = alpha2[e] * (a2_hat[p] . w2_hat[e]^T),  alpha2[e] = fl32((*g2) * gw2[e])
 * then out[t] = sum_j topk_w[t][j] * d[inv_pos[t*topk + j]] (+ d of the shared
 * pair with weight 1), summed in FP32 in the order j = 0..topk-1, shared last,
 * rows with inv_pos = -1 skipped.  out is [T][H] bfloat16 (out_dtype
 * NVFP4_BF16, round to nearest even: the bf16-only output of vLLM PR #29242,
 * "Force bf16 only") or float32 (NVFP4_F32, the same sums unrounded).
 * a2_deq (optional): the a2_deq output of grouped_gemm1_swiglu, read instead
 * of a2_q/a2_sf (which may then be NULL). */
int grouped_gemm2_combine(const nvfp4_moe_dims* dims, const uint8_t* a2_q, const uint8_t* a2_sf,
                          const uint16_t* a2_deq, const float* g2, const int32_t* expert_offsets,
                          const int32_t* inv_pos,
                          const int32_t* plan, const float* topk_w, const uint8_t* w2_prep,
                          const float* gw2, void* out, int out_dtype, void* ws, size_t ws_bytes,
                          void* stream);

/* GEMM1, weight-only variant (W4A16, the Marlin-style dequantising path of
 * FlashInfer #2723, "Speed Comparison"; unsloth PR #10417, "Why it
 * matters"): activations stay bfloat16 (x [T][H]), weights are dequantised
 * in-kernel, alpha1[e] = gw13[e], and the intermediate a2 [P][I] is h rounded
 * to bfloat16 (nearest even). */
int grouped_gemm1_swiglu_w4a16(const nvfp4_moe_dims* dims, const uint16_t* x,
                               const int32_t* sorted_pair, const int32_t* expert_offsets,
                               const int32_t* plan, const uint8_t* w13_prep, const float* gw13,
                               uint16_t* a2, void* stream);

/* GEMM2 + combine, weight-only variant: a2 bfloat16 [P][I], alpha2[e] =
 * gw2[e]; combine and output as grouped_gemm2_combine. */
int grouped_gemm2_combine_w4a16(const nvfp4_moe_dims* dims, const uint16_t* a2,
                                const int32_t* expert_offsets, const int32_t* inv_pos,
                                const int32_t* plan, const float* topk_w, const uint8_t* w2_prep,
                                const float* gw2, void* out, int out_dtype, void* ws,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Mixture-of-experts layer in OCP MXFP4 (grouped GEMMs on the scaled FP4      */
/* matrix instruction).                                                       */
/* ------------------------------------------------------------------------ */
/* The emulation backend's OCP MX path runs the experts of MXFP4 models (vLLM
 * PR #35737, "Purpose"); here the same layer as the NVFP4 W4A4 path with
 * MXFP4 (E2M1 codes, one E8M0 exponent byte per 32 elements, no global scale,
 * the rules of mxfp4_quantize) for the activations, the expert weights and
 * the intermediate.  The block scales are powers of two per 32, exactly what
 * CDNA4's scaled FP4 matrix instruction takes, so codes are multiplied as
 * stored.  The layer:
 *   mxfp4_quantize(x)                 a1: codes [T][H/2], exponents [T][H/32]
 *   moe_align(dims, topk_ids, ...)    the permutation and tile plan
 *                                     (both in one call:
 *                                     moe_mxfp4_quantize_and_align)
 *   grouped_gemm1_swiglu_mxfp4        per row p of expert e (token t):
 *                                     h = silu(c[0:I]) * c[I:2I],
 *                                     c = a1_hat[t] . w13_hat[e]^T (FP32),
 *                                     a2 row p = MXFP4(h) (block scale from h)
 *   grouped_gemm2_combine_mxfp4       d[p] = a2_hat[p] . w2_hat[e]^T, then
 *                                     out as grouped_gemm2_combine.
 * Expert weights (canonical MXFP4, q [S][N][K/2], ex [S][N][K/32], S = E +
 * shared; which = 13: [2I][H] rows [0, I) gate, [I, 2I) up; which = 2:
 * [H][I]) are rearranged offline by mxfp4_prep_expert_weights into prep
 * (mxfp4_prep_expert_weights_size bytes, 16-byte aligned, opaque).
 * a1_q/a2_q must be 16-byte and a1_e/a2_e 4-byte aligned; T*H/2, P*I/2 and
 * I*H must stay below 2^31 (ESHAPE otherwise).  ws: grouped_gemm_workspace_size
 * bytes (the FP32 rows the combine reads). */
size_t mxfp4_prep_expert_weights_size(const nvfp4_moe_dims* dims, int which);
int mxfp4_prep_expert_weights(const nvfp4_moe_dims* dims, int which, const uint8_t* q, const uint8_t* ex,
                              uint8_t* prep, void* stream);
int grouped_gemm1_swiglu_mxfp4(const nvfp4_moe_dims* dims, const uint8_t* a1_q, const uint8_t* a1_e,
                               const int32_t* sorted_pair, const int32_t* expert_offsets, const int32_t* plan,
                               const uint8_t* w13_prep, uint8_t* a2_q, uint8_t* a2_e, void* stream);
int grouped_gemm2_combine_mxfp4(const nvfp4_moe_dims* dims, const uint8_t* a2_q, const uint8_t* a2_e,
                                const int32_t* expert_offsets, const int32_t* inv_pos, const int32_t* plan,
                                const float* topk_w, const uint8_t* w2_prep, void* out, int out_dtype, void* ws,
                                size_t ws_bytes, void* stream);
/* The layer's first two steps in one call: the same results, bit for bit,
 * as mxfp4_quantize(x, NVFP4_BF16, T, H, H, a1_q, a1_e, ...) followed by
 * moe_align(dims, topk_ids, ...), with those calls' argument contracts (x
 * bfloat16 [T][H] 16-byte aligned, a1_q [T][H/2] 4-byte aligned, a1_e
 * [T][H/32]; ws: moe_align_workspace_size(dims) bytes).  MXFP4 has no global
 * scale, so the two steps are independent: when the pairs fit one workgroup
 * (P <= 4096) they share one launch; otherwise the quantisation runs beside
 * the pair scatter, after the count and scan launches.  Errors: as for
 * those calls, and NVFP4_ESHAPE when T*H >= 2^31. */
int moe_mxfp4_quantize_and_align(const nvfp4_moe_dims* dims, const uint16_t* x, uint8_t* a1_q, uint8_t* a1_e,
                                 const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pair,
                                 int32_t* inv_pos, int32_t* plan, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The grouped GEMMs in two parts, for two streams.                          */
/* ------------------------------------------------------------------------ */
/* A scheduling interface, not an operation of its own (the pages define
 * none): when the pairs are few per expert on average but some expert may
 * still hold more than 64 rows (the 512-expert layer with a shared expert of
 * FlashInfer #2723, "Model"), the GEMMs run the short experts and the tall
 * ones as separate launches that write disjoint rows.  A caller with a second
 * stream can run the two side by side:
 *   part 1 (short experts) and part 2 (tall experts) of GEMM1, then of GEMM2,
 *   each part's GEMM2 after the same part's GEMM1 (it reads only the a2 rows
 *   that part wrote), and part 3 (the combine) after both parts' GEMM2.
 * Each *_part call takes the arguments of the call it is named after, plus
 * part: 0 = the whole call (the same as the call itself), 1 = the short
 * experts' rows, 2 = the tall experts' rows, 3 (GEMM2 calls only) = the
 * combine alone.  Parts 1 and 2 write the same values, bit for bit, as part 0
 * writes to those rows; for dimensions that do not run in two parts (see
 * grouped_gemm_runs_in_parts, and W4A4 without the f16 activation copies),
 * part 1 is the whole GEMM and part 2 launches nothing.  Errors: those of the
 * named call, and NVFP4_EINVAL for a part outside 0..2 (GEMM1) or 0..3 (GEMM2).
 * The library creates no stream or event: ordering the parts is the caller's
 * (events between its streams). */

/* 1 when these dimensions run the grouped GEMMs in two parts (then a second
 * stream can overlap them), else 0 (also 0 for invalid dims). */
int grouped_gemm_runs_in_parts(const nvfp4_moe_dims* dims);
int grouped_gemm1_swiglu_part(const nvfp4_moe_dims* dims, const uint8_t* a1_q, const uint8_t* a1_sf,
                              const uint16_t* a1_deq, const float* g1, const int32_t* sorted_pair,
                              const int32_t* expert_offsets, const int32_t* plan, const uint8_t* w13_prep,
                              const float* gw13, const float* g2, uint8_t* a2_q, uint8_t* a2_sf,
                              uint16_t* a2_deq, int part, void* stream);
int grouped_gemm2_combine_part(const nvfp4_moe_dims* dims, const uint8_t* a2_q, const uint8_t* a2_sf,
                               const uint16_t* a2_deq, const float* g2, const int32_t* expert_offsets,
                               const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                               const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype, void* ws,
                               size_t ws_bytes, int part, void* stream);
int grouped_gemm1_swiglu_w4a16_part(const nvfp4_moe_dims* dims, const uint16_t* x, const int32_t* sorted_pair,
                                    const int32_t* expert_offsets, const int32_t* plan, const uint8_t* w13_prep,
                                    const float* gw13, uint16_t* a2, int part, void* stream);
int grouped_gemm2_combine_w4a16_part(const nvfp4_moe_dims* dims, const uint16_t* a2, const int32_t* expert_offsets,
                                     const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                                     const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype, void* ws,
                                     size_t ws_bytes, int part, void* stream);
int grouped_gemm1_swiglu_mxfp4_part(const nvfp4_moe_dims* dims, const uint8_t* a1_q, const uint8_t* a1_e,
                                    const int32_t* sorted_pair, const int32_t* expert_offsets, const int32_t* plan,
                                    const uint8_t* w13_prep, uint8_t* a2_q, uint8_t* a2_e, int part, void* stream);
int grouped_gemm2_combine_mxfp4_part(const nvfp4_moe_dims* dims, const uint8_t* a2_q, const uint8_t* a2_e,
                                     const int32_t* expert_offsets, const int32_t* inv_pos, const int32_t* plan,
                                     const float* topk_w, const uint8_t* w2_prep, void* out, int out_dtype,
                                     void* ws, size_t ws_bytes, int part, void* stream);

/* ------------------------------------------------------------------------ */
/* GEMM2 + combine without allocation.                                       */
/* ------------------------------------------------------------------------ */
/* For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation and results, bit for bit, as
 * grouped_gemm2_combine with the same arguments, except that the per-row
 * FP32 down-projection outputs live in a static scratch array inside the
 * library (one per GPU, held until the process ends) instead of a
 * caller-owned workspace.  Limit: P * H * 4 bytes <=
 * grouped_gemm2_combine_noalloc_max_bytes() (48 MiB: P * H <= 12,582,912,
 * e.g. every decode-shaped batch of this header's examples, T * topk up to
 * 6144 rows at H = 2048); larger shapes return NVFP4_EWORKSPACE with the
 * needed and available sizes.  The call allocates and frees nothing; on its
 * first call on a device it looks up that device's copy of the array
 * (hipGetSymbolAddress).  Every call on a GPU shares that GPU's array, which
 * keeps the last call's contents (nothing in it needs clearing: each call
 * writes every row it reads): calls that overlap on one GPU (concurrent
 * streams, or threads on one device) race and must be serialised by the
 * caller. */
size_t grouped_gemm2_combine_noalloc_max_bytes(void);
int grouped_gemm2_combine_noalloc(const nvfp4_moe_dims* dims, const uint8_t* a2_q, const uint8_t* a2_sf,
                                  const uint16_t* a2_deq, const float* g2, const int32_t* expert_offsets,
                                  const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                                  const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MOE_H */
