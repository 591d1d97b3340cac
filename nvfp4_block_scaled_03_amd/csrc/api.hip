// C ABI of libnvfp4moe.so: host-side validation, error reporting and kernel
// dispatch.  Every argument is checked before anything is launched; a failed
// check returns a negative status, launches nothing and leaves a thread-local
// message naming the call and the offending values (num_experts, M, N, K and
// the workspace size for the GEMMs, like the grouped-GEMM initialisation error
// of vLLM PR #29242, review of nvfp4_blockwise_moe_kernel.cu).
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/nvfp4_moe.h"
#include "launch.h"
#include "mx.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return NVFP4_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NVFP4_ELAUNCH, "%s: ELAUNCH %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

// Shared validation of the layer dimensions.
int check_dims(const nvfp4_moe_dims* d, const char* what) {
  if (!d) return fail(NVFP4_EINVAL, "%s: EINVAL dims is NULL", what);
  if (d->T < 0 || d->topk < 1 || d->E < 1 || d->topk > d->E || d->H <= 0 || d->I <= 0 ||
      (d->shared != 0 && d->shared != 1))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE T=%d topk=%d num_experts=%d H=%d I=%d shared=%d", what,
                d->T, d->topk, d->E, d->H, d->I, d->shared);
  if (d->H % 128 || d->I % 128)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE H=%d and I=%d must be multiples of 128", what, d->H, d->I);
  if (d->E + d->shared > nvfp4::kMaxExperts)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE num_experts=%d (+%d shared) exceeds %d", what, d->E,
                d->shared, nvfp4::kMaxExperts);
  const int64_t P = (int64_t)d->T * d->topk + (int64_t)d->shared * d->T;
  if (P > ((int64_t)1 << 24))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE pairs=%lld exceeds 2^24", what, (long long)P);
  return NVFP4_OK;
}

int64_t pairs(const nvfp4_moe_dims* d) {
  return (int64_t)d->T * d->topk + (int64_t)d->shared * d->T;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_MOE_ABI_VERSION; }

const char* nvfp4_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------ scales
size_t nvfp4_global_scale_workspace_size(int64_t batches, int64_t n) {
  if (batches <= 0 || n < 0) return 0;
  return nvfp4::global_scale_ws_bytes(batches, n);
}

int nvfp4_global_scale(const void* x, int dtype, int64_t batches, int64_t n, float* g, void* ws,
                       size_t ws_bytes, void* stream) {
  const char* W = "nvfp4_global_scale";
  if (dtype != NVFP4_BF16 && dtype != NVFP4_F32)
    return fail(NVFP4_EINVAL, "%s: EINVAL dtype=%d", W, dtype);
  if (batches < 0 || n < 0 || n % 8 || batches > 65535)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE batches=%lld n=%lld (n %% 8 == 0, batches <= 65535)", W,
                (long long)batches, (long long)n);
  if (batches == 0) return ok();
  if (!g || (n > 0 && !x)) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(g, 4) || !aligned(ws, 4))
    return fail(NVFP4_EINVAL, "%s: EINVAL misaligned x, g or ws", W);
  const size_t need = nvfp4_global_scale_workspace_size(batches, n);
  if (ws_bytes < need || !ws)
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE workspace_size=%zu needed=%zu", W, ws_bytes, need);
  return launched(nvfp4::launch_global_scale(x, dtype, batches, n, g, ws, S(stream)), W);
}

int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, const float* g,
                   int64_t rows_per_g, uint8_t* q, uint8_t* sf, uint16_t* x_deq, void* stream) {
  const char* W = "nvfp4_quantize";
  if (dtype != NVFP4_BF16 && dtype != NVFP4_F32)
    return fail(NVFP4_EINVAL, "%s: EINVAL dtype=%d", W, dtype);
  if (rows < 0 || K <= 0 || K % 16 || ldx < K || ldx % 8 || rows_per_g < 1)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE rows=%lld K=%lld ldx=%lld rows_per_g=%lld", W,
                (long long)rows, (long long)K, (long long)ldx, (long long)rows_per_g);
  if ((rows * (K / 8) + 255) / 256 > 0x7FFFFFFFLL)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE rows=%lld K=%lld too large", W, (long long)rows,
                (long long)K);
  if (rows == 0) return ok();
  if (!x || !g || !q || !sf) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(g, 4) || !aligned(x_deq, 16))
    return fail(NVFP4_EINVAL, "%s: EINVAL misaligned pointer (x, x_deq 16 B, q 4 B)", W);
  return launched(nvfp4::launch_quantize(x, dtype, rows, K, ldx, g, rows_per_g, q, sf, x_deq,
                                         S(stream)), W);
}

// ------------------------------------------------------------------ router
int moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t topk, int32_t* ids,
                   float* weights, void* stream) {
  const char* W = "moe_route_topk";
  if (T < 0 || E < 1 || E > 1024 || topk < 1 || topk > E || topk > 32)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE T=%d num_experts=%d topk=%d", W, T, E, topk);
  if (T == 0) return ok();
  if (!logits || !ids || !weights) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  return launched(nvfp4::launch_route_topk(logits, T, E, topk, ids, weights, S(stream)), W);
}

// ------------------------------------------------------------------ align
size_t moe_align_workspace_size(const nvfp4_moe_dims* d) {
  if (check_dims(d, "moe_align_workspace_size")) return 0;
  const nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  return nvfp4::align_ws_bytes(a);
}

size_t moe_align_plan_size(const nvfp4_moe_dims* d) {
  if (check_dims(d, "moe_align_plan_size")) return 0;
  const nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  return nvfp4::align_plan_ints(a) * sizeof(int32_t);
}

int moe_align(const nvfp4_moe_dims* d, const int32_t* topk_ids, int32_t* expert_offsets,
              int32_t* sorted_pair, int32_t* inv_pos, int32_t* plan, void* ws, size_t ws_bytes,
              void* stream) {
  const char* W = "moe_align";
  if (int r = check_dims(d, W)) return r;
  if (d->T == 0) return ok();
  const nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  if (!expert_offsets || !plan) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (a.P > 0 && (!sorted_pair || !inv_pos || (d->T * d->topk > 0 && !topk_ids)))
    return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  const size_t need = nvfp4::align_ws_bytes(a);
  if (ws_bytes < need || (need && !ws))
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld workspace_size=%zu needed=%zu",
                W, d->E, (long long)a.P, ws_bytes, need);
  return launched(nvfp4::launch_align(a, topk_ids, expert_offsets, sorted_pair, inv_pos, plan, ws,
                                      S(stream)), W);
}

int moe_scale_and_align(const nvfp4_moe_dims* d, const uint16_t* x, float* g1, void* gs_ws,
                        size_t gs_ws_bytes, const int32_t* topk_ids, int32_t* expert_offsets,
                        int32_t* sorted_pair, int32_t* inv_pos, int32_t* plan, void* ws,
                        size_t ws_bytes, void* stream) {
  const char* W = "moe_scale_and_align";
  if (int r = check_dims(d, W)) return r;
  if (d->T == 0) return ok();
  nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  a.H = d->H;
  if (!expert_offsets || !plan || !g1) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (a.P > 0 && (!sorted_pair || !inv_pos || (d->T * d->topk > 0 && !topk_ids) || !x))
    return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(g1, 4) || !aligned(gs_ws, 4))
    return fail(NVFP4_EINVAL, "%s: EINVAL misaligned x, g1 or gs_ws", W);
  const size_t gs_need = nvfp4_global_scale_workspace_size(1, (int64_t)d->T * d->H);
  if (gs_ws_bytes < gs_need || !gs_ws)
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE global-scale workspace_size=%zu needed=%zu", W,
                gs_ws_bytes, gs_need);
  const size_t need = nvfp4::align_ws_bytes(a);
  if (ws_bytes < need || (need && !ws))
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld workspace_size=%zu needed=%zu",
                W, d->E, (long long)a.P, ws_bytes, need);
  return launched(nvfp4::launch_scale_and_align(a, x, g1, gs_ws, topk_ids, expert_offsets, sorted_pair,
                                                inv_pos, plan, ws, S(stream)), W);
}

int moe_route_and_align(const nvfp4_moe_dims* d, const float* logits, int32_t* topk_ids,
                        float* topk_w, int32_t* expert_offsets, int32_t* sorted_pair, int32_t* inv_pos,
                        int32_t* plan, void* ws, size_t ws_bytes, void* stream) {
  const char* W = "moe_route_and_align";
  if (int r = check_dims(d, W)) return r;
  if (d->T == 0) return ok();
  if (d->topk > 32)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE num_experts=%d topk=%d (router: topk <= 32)", W, d->E, d->topk);
  nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  if (!expert_offsets || !plan) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (a.P > 0 && (!sorted_pair || !inv_pos)) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (d->T > 0 && (!logits || !topk_ids || !topk_w)) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  const size_t need = nvfp4::align_ws_bytes(a);
  if (ws_bytes < need || (need && !ws))
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld workspace_size=%zu needed=%zu",
                W, d->E, (long long)a.P, ws_bytes, need);
  return launched(nvfp4::launch_route_and_align(a, logits, topk_ids, topk_w, expert_offsets, sorted_pair,
                                                inv_pos, plan, ws, S(stream)),
                  W);
}

int moe_quantize_and_align(const nvfp4_moe_dims* d, const uint16_t* x, float* g1, void* gs_ws,
                           size_t gs_ws_bytes, uint8_t* a1_q, uint8_t* a1_sf, uint16_t* a1_deq,
                           const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pair,
                           int32_t* inv_pos, int32_t* plan, void* ws, size_t ws_bytes, void* stream) {
  const char* W = "moe_quantize_and_align";
  if (int r = check_dims(d, W)) return r;
  if (d->T == 0) return ok();
  nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  a.H = d->H;
  if (!expert_offsets || !plan || !g1) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (a.P > 0 && (!sorted_pair || !inv_pos || (d->T * d->topk > 0 && !topk_ids) || !x))
    return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (d->T > 0 && (!a1_q || !a1_sf)) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(g1, 4) || !aligned(gs_ws, 4) || !aligned(a1_q, 4) ||
      !aligned(a1_deq, 16))
    return fail(NVFP4_EINVAL, "%s: EINVAL misaligned x, g1, gs_ws, a1_q or a1_deq", W);
  const size_t gs_need = nvfp4_global_scale_workspace_size(1, (int64_t)d->T * d->H);
  if (gs_ws_bytes < gs_need || !gs_ws)
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE global-scale workspace_size=%zu needed=%zu", W,
                gs_ws_bytes, gs_need);
  const size_t need = nvfp4::align_ws_bytes(a);
  if (ws_bytes < need || (need && !ws))
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld workspace_size=%zu needed=%zu",
                W, d->E, (long long)a.P, ws_bytes, need);
  return launched(nvfp4::launch_quantize_and_align(a, x, g1, gs_ws, a1_q, a1_sf, a1_deq, topk_ids,
                                                   expert_offsets, sorted_pair, inv_pos, plan, ws,
                                                   S(stream)),
                  W);
}

int moe_mxfp4_quantize_and_align(const nvfp4_moe_dims* d, const uint16_t* x, uint8_t* a1_q, uint8_t* a1_e,
                                 const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pair,
                                 int32_t* inv_pos, int32_t* plan, void* ws, size_t ws_bytes, void* stream) {
  const char* W = "moe_mxfp4_quantize_and_align";
  if (int r = check_dims(d, W)) return r;
  if ((int64_t)d->T * d->H >= (int64_t(1) << 31))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE T=%d H=%d too large", W, d->T, d->H);
  if (d->T == 0) return ok();
  nvfp4::AlignShape a = nvfp4::align_shape(d->T, d->topk, d->E, d->shared);
  a.H = d->H;
  if (!expert_offsets || !plan || !x || !a1_q || !a1_e) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (a.P > 0 && (!sorted_pair || !inv_pos || (d->T * d->topk > 0 && !topk_ids)))
    return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(a1_q, 4))
    return fail(NVFP4_EINVAL, "%s: EINVAL misaligned x or a1_q", W);
  const size_t need = nvfp4::align_ws_bytes(a);
  if (ws_bytes < need || (need && !ws))
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld workspace_size=%zu needed=%zu",
                W, d->E, (long long)a.P, ws_bytes, need);
  return launched(nvfp4::launch_mx_quantize_and_align(a, x, a1_q, a1_e, topk_ids, expert_offsets, sorted_pair,
                                                      inv_pos, plan, ws, S(stream)),
                  W);
}

// ------------------------------------------------------------------ dense linear
namespace {
// Workspace of nvfp4_linear*: 256-byte aligned sub-buffers in this order.
struct LinearWs {
  size_t g, gs, offsets, sorted_pair, inv_pos, plan, align, a_q, a_sf, a_deq, total;
};
size_t up256(size_t b) { return (b + 255) & ~size_t(255); }
bool linear_shape_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 0 && M <= (int64_t(1) << 24) && N > 0 && K > 0 && N % 128 == 0 && K % 128 == 0 &&
         N <= (int64_t(1) << 20) && K <= (int64_t(1) << 20);
}
LinearWs linear_ws(int64_t M, int64_t N, int64_t K, bool w4a4) {
  const nvfp4::AlignShape a = nvfp4::align_shape((int)M, 1, 1, 0);
  LinearWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += up256(bytes); return at; };
  w.g = take(w4a4 ? 4 : 0);
  w.gs = take(w4a4 ? nvfp4_global_scale_workspace_size(1, std::max<int64_t>(M * K, 8)) : 0);
  w.offsets = take(2 * sizeof(int32_t));
  w.sorted_pair = take((size_t)std::max<int64_t>(M, 1) * 4);
  w.inv_pos = take((size_t)std::max<int64_t>(M, 1) * 4);
  w.plan = take(nvfp4::align_plan_ints(a) * 4);
  w.align = take(nvfp4::align_ws_bytes(a));
  w.a_q = take(w4a4 ? (size_t)M * (K / 2) : 0);
  w.a_sf = take(w4a4 ? (size_t)M * (K / 16) : 0);
  w.a_deq = take(w4a4 && nvfp4::prefers_decoded((int)M, 1, 1, 0) ? (size_t)M * K * 2 : 0);
  w.total = o;
  return w;
}

int linear_run(const char* W, bool w4a4, const uint16_t* x, int64_t M, int64_t N, int64_t K,
               const uint8_t* w_prep, const float* gw, void* out, int out_dtype, void* ws,
               size_t ws_bytes, void* stream) {
  if (!linear_shape_ok(M, N, K))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE M=%lld N=%lld K=%lld (N, K multiples of 128)", W, (long long)M,
                (long long)N, (long long)K);
  if (out_dtype != 0 && out_dtype != 1) return fail(NVFP4_EINVAL, "%s: EINVAL out_dtype=%d", W, out_dtype);
  const LinearWs L = linear_ws(M, N, K, w4a4);
  if (ws_bytes < L.total || !ws)
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=1 M=%lld N=%lld K=%lld workspace_size=%zu needed=%zu",
                W, (long long)M, (long long)N, (long long)K, ws_bytes, L.total);
  if (M == 0) return ok();
  if (!x || !w_prep || !gw || !out) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(w_prep, 16) || !aligned(ws, 256) || !aligned(out, 16))
    return fail(NVFP4_EINVAL, "%s: EINVAL x, w_prep and out 16-byte, ws 256-byte aligned", W);
  uint8_t* b = static_cast<uint8_t*>(ws);
  nvfp4::AlignShape a = nvfp4::align_shape((int)M, 1, 1, 0);
  a.H = (int)K;
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* sp = reinterpret_cast<int32_t*>(b + L.sorted_pair);
  int32_t* inv = reinterpret_cast<int32_t*>(b + L.inv_pos);
  int32_t* plan = reinterpret_cast<int32_t*>(b + L.plan);
  nvfp4::LinearArgs la{};
  la.M = M;
  la.N = N;
  la.K = K;
  la.w4a4 = w4a4;
  la.plan = plan;
  la.w_prep = w_prep;
  la.g_w = gw;
  la.out = out;
  la.out_dtype = out_dtype;
  hipError_t e;
  if (w4a4) {
    float* g = reinterpret_cast<float*>(b + L.g);
    uint8_t* aq = b + L.a_q;
    uint8_t* asf = b + L.a_sf;
    uint16_t* adeq = nvfp4::prefers_decoded((int)M, 1, 1, 0) ? reinterpret_cast<uint16_t*>(b + L.a_deq)
                                                              : nullptr;
    e = nvfp4::launch_quantize_and_align(a, x, g, b + L.gs, aq, asf, adeq, nullptr, offsets, sp, inv, plan,
                                         b + L.align, S(stream));
    la.g_a = g;
    la.a_q = aq;
    la.a_sf = asf;
    la.a_h = adeq;
  } else {
    e = nvfp4::launch_align(a, nullptr, offsets, sp, inv, plan, b + L.align, S(stream));
    la.a_h = x;
  }
  if (e != hipSuccess) return launched(e, W);
  return launched(nvfp4::launch_linear(la, S(stream)), W);
}
}  // namespace

size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int w4a4) {
  if (!linear_shape_ok(M, N, K)) return 0;
  return linear_ws(M, N, K, w4a4 != 0).total;
}

int nvfp4_linear(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_prep,
                 const float* gw, void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  return linear_run("nvfp4_linear", true, x, M, N, K, w_prep, gw, out, out_dtype, ws, ws_bytes, stream);
}

int nvfp4_linear_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_prep,
                       const float* gw, void* out, int out_dtype, void* ws, size_t ws_bytes,
                       void* stream) {
  return linear_run("nvfp4_linear_w4a16", false, x, M, N, K, w_prep, gw, out, out_dtype, ws, ws_bytes,
                    stream);
}

// ------------------------------------------------------------------ MXFP4
int mxfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, uint8_t* q, uint8_t* ex,
                   void* stream) {
  const char* W = "mxfp4_quantize";
  if (dtype != 0 && dtype != 1) return fail(NVFP4_EINVAL, "%s: EINVAL dtype=%d", W, dtype);
  if (rows < 0 || K <= 0 || K % 32 || ldx < K || ldx % 8)
    return fail(NVFP4_ESHAPE, "%s: ESHAPE rows=%lld K=%lld ldx=%lld", W, (long long)rows, (long long)K,
                (long long)ldx);
  if (rows * K >= (int64_t(1) << 31))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE rows=%lld K=%lld too large", W, (long long)rows, (long long)K);
  if (rows == 0) return ok();
  if (!x || !q || !ex) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(q, 4)) return fail(NVFP4_EINVAL, "%s: EINVAL misaligned x or q", W);
  return launched(nvfp4::launch_mx_quantize(x, dtype, rows, K, ldx, q, ex, S(stream)), W);
}

size_t mxfp4_prep_weights_size(int64_t N, int64_t K) {
  if (!linear_shape_ok(1, N, K)) return 0;
  return nvfp4::mx_prep_bytes(N, K);
}

int mxfp4_prep_weights(int64_t N, int64_t K, const uint8_t* q, const uint8_t* ex, uint8_t* prep,
                       void* stream) {
  const char* W = "mxfp4_prep_weights";
  if (!linear_shape_ok(1, N, K))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE N=%lld K=%lld (multiples of 128)", W, (long long)N, (long long)K);
  if (!q || !ex || !prep) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(q, 16) || !aligned(prep, 16))
    return fail(NVFP4_EINVAL, "%s: EINVAL q and prep must be 16-byte aligned", W);
  return launched(nvfp4::launch_mx_prep(N, K, q, ex, prep, S(stream)), W);
}

namespace {
// Workspace of mxfp4_linear: the activation operand's codes, then its scale
// words (rows padded to whole tiles).
size_t mx_ws_codes(int64_t M, int64_t K) { return up256((size_t)nvfp4::mx_rows_pad(M) * (K / 2)); }
}  // namespace

size_t mxfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (!linear_shape_ok(M, N, K)) return 0;
  return mx_ws_codes(M, K) + up256((size_t)nvfp4::mx_rows_pad(M) * (K / 32));
}

int mxfp4_linear(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_prep, void* out,
                 int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  const char* W = "mxfp4_linear";
  if (!linear_shape_ok(M, N, K) || nvfp4::mx_rows_pad(M) * K >= (int64_t(1) << 31) ||
      (N * K / 32) * 17 >= (int64_t(1) << 32))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE M=%lld N=%lld K=%lld (N, K multiples of 128; M K < 2^31, prepared "
                "weight < 4 GiB)", W, (long long)M, (long long)N, (long long)K);
  if (out_dtype != 0 && out_dtype != 1) return fail(NVFP4_EINVAL, "%s: EINVAL out_dtype=%d", W, out_dtype);
  const size_t need = mxfp4_linear_workspace_size(M, N, K);
  if (ws_bytes < need || (M > 0 && !ws))
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE M=%lld N=%lld K=%lld workspace_size=%zu needed=%zu", W,
                (long long)M, (long long)N, (long long)K, ws_bytes, need);
  if (M == 0) return ok();
  if (!x || !w_prep || !out) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(x, 16) || !aligned(w_prep, 16) || !aligned(ws, 256))
    return fail(NVFP4_EINVAL, "%s: EINVAL x and w_prep 16-byte, ws 256-byte aligned", W);
  uint8_t* aq = static_cast<uint8_t*>(ws);
  uint8_t* ae = aq + mx_ws_codes(M, K);
  hipError_t e = nvfp4::launch_mx_quantize_operand(x, M, K, aq, ae, S(stream));
  if (e != hipSuccess) return launched(e, W);
  return launched(nvfp4::launch_mx_gemm(aq, ae, M, N, K, w_prep, out, out_dtype, S(stream)), W);
}

// ------------------------------------------------------------------ weights
size_t nvfp4_prep_weights_size(const nvfp4_moe_dims* d, int which) {
  if (check_dims(d, "nvfp4_prep_weights_size") || (which != 13 && which != 2)) return 0;
  const int64_t slots = d->E + d->shared;
  return which == 13 ? nvfp4::prep_bytes(slots, 2 * (int64_t)d->I, d->H)
                     : nvfp4::prep_bytes(slots, d->H, d->I);
}

int nvfp4_prep_weights(const nvfp4_moe_dims* d, int which, const uint8_t* q, const uint8_t* sf,
                       uint8_t* prep, void* stream) {
  const char* W = "nvfp4_prep_weights";
  if (int r = check_dims(d, W)) return r;
  if (which != 13 && which != 2) return fail(NVFP4_EINVAL, "%s: EINVAL which=%d (13 or 2)", W, which);
  if (!q || !sf || !prep) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(q, 16) || !aligned(prep, 16))
    return fail(NVFP4_EINVAL, "%s: EINVAL q and prep must be 16-byte aligned", W);
  const int64_t slots = d->E + d->shared;
  const int64_t N = which == 13 ? 2 * (int64_t)d->I : d->H;
  const int64_t K = which == 13 ? d->H : d->I;
  return launched(nvfp4::launch_prep(slots, N, K, which == 13 ? d->I : 0, q, sf, prep, S(stream)), W);
}

// ------------------------------------------------------------------ GEMMs
int grouped_gemm_prefers_decoded(const nvfp4_moe_dims* d) {
  if (check_dims(d, "grouped_gemm_prefers_decoded")) return 0;
  return nvfp4::prefers_decoded(d->T, d->topk, d->E, d->shared) ? 1 : 0;
}

int grouped_gemm_runs_in_parts(const nvfp4_moe_dims* d) {
  if (check_dims(d, "grouped_gemm_runs_in_parts")) return 0;
  return nvfp4::split_experts(nvfp4::align_shape(d->T, d->topk, d->E, d->shared)) ? 1 : 0;
}

size_t grouped_gemm_workspace_size(const nvfp4_moe_dims* d) {
  if (check_dims(d, "grouped_gemm_workspace_size")) return 0;
  return (size_t)pairs(d) * (size_t)d->H * sizeof(float);
}

static int gemm_fail_shape(const char* W, const nvfp4_moe_dims* d, int N, int K, size_t ws) {
  return fail(NVFP4_EINVAL, "%s: EINVAL null or misaligned pointer num_experts=%d M=%lld N=%d K=%d "
              "workspace_size=%zu", W, d->E + d->shared, (long long)pairs(d), N, K, ws);
}

static nvfp4::GemmArgs gemm_args(const nvfp4_moe_dims* d) {
  nvfp4::GemmArgs a{};
  a.T = d->T;
  a.topk = d->topk;
  a.E = d->E;
  a.shared = d->shared;
  a.H = d->H;
  a.I = d->I;
  a.P = pairs(d);
  return a;
}

static int grouped_gemm1_swiglu_impl(const char* W, int part, const nvfp4_moe_dims* d, const uint8_t* a1_q,
                                     const uint8_t* a1_sf, const uint16_t* a1_deq, const float* g1,
                                     const int32_t* sorted_pair, const int32_t* expert_offsets,
                                     const int32_t* plan, const uint8_t* w13_prep, const float* gw13,
                                     const float* g2, uint8_t* a2_q, uint8_t* a2_sf, uint16_t* a2_deq,
                                     void* stream) {
  if (int r = check_dims(d, W)) return r;
  if (d->T == 0) return ok();
  if ((!a1_deq && (!a1_q || !a1_sf)) || !g1 || !sorted_pair || !expert_offsets || !plan ||
      !w13_prep || !gw13 || !g2 || !a2_q || !a2_sf || !aligned(a1_q, 16) || !aligned(a1_sf, 2) ||
      !aligned(a1_deq, 16) || !aligned(a2_deq, 2) || !aligned(w13_prep, 16))
    return gemm_fail_shape(W, d, 2 * d->I, d->H, 0);
  nvfp4::GemmArgs a = gemm_args(d);
  a.offsets = expert_offsets;
  a.sorted_pair = sorted_pair;
  a.plan = plan;
  a.a_q = a1_q;
  a.a_sf = a1_sf;
  a.a_h = a1_deq;
  a.g_a = g1;
  a.w_prep = w13_prep;
  a.g_w = gw13;
  a.g2 = g2;
  a.out_q = a2_q;
  a.out_sf = a2_sf;
  a.out_h = a2_deq;
  a.part = part;
  return launched(nvfp4::launch_gemm1(a, true, S(stream)), W);
}

int grouped_gemm1_swiglu(const nvfp4_moe_dims* d, const uint8_t* a1_q, const uint8_t* a1_sf,
                         const uint16_t* a1_deq, const float* g1, const int32_t* sorted_pair,
                         const int32_t* expert_offsets, const int32_t* plan, const uint8_t* w13_prep,
                         const float* gw13, const float* g2, uint8_t* a2_q, uint8_t* a2_sf, uint16_t* a2_deq,
                         void* stream) {
  return grouped_gemm1_swiglu_impl("grouped_gemm1_swiglu", nvfp4::kPartAll, d, a1_q, a1_sf, a1_deq, g1,
                                   sorted_pair, expert_offsets, plan, w13_prep, gw13, g2, a2_q, a2_sf, a2_deq,
                                   stream);
}

int grouped_gemm1_swiglu_part(const nvfp4_moe_dims* d, const uint8_t* a1_q, const uint8_t* a1_sf,
                              const uint16_t* a1_deq, const float* g1, const int32_t* sorted_pair,
                              const int32_t* expert_offsets, const int32_t* plan, const uint8_t* w13_prep,
                              const float* gw13, const float* g2, uint8_t* a2_q, uint8_t* a2_sf,
                              uint16_t* a2_deq, int part, void* stream) {
  if (part < 0 || part > 2)
    return fail(NVFP4_EINVAL, "%s: EINVAL part=%d (0..2)", "grouped_gemm1_swiglu_part", part);
  return grouped_gemm1_swiglu_impl("grouped_gemm1_swiglu_part", part, d, a1_q, a1_sf, a1_deq, g1, sorted_pair,
                                   expert_offsets, plan, w13_prep, gw13, g2, a2_q, a2_sf, a2_deq, stream);
}

static int grouped_gemm1_swiglu_w4a16_impl(const char* W, int part, const nvfp4_moe_dims* d,
                                           const uint16_t* x, const int32_t* sorted_pair,
                                           const int32_t* expert_offsets, const int32_t* plan,
                                           const uint8_t* w13_prep, const float* gw13, uint16_t* a2,
                                           void* stream) {
  if (int r = check_dims(d, W)) return r;
  if (d->T == 0) return ok();
  if (!x || !sorted_pair || !expert_offsets || !plan || !w13_prep || !gw13 || !a2 ||
      !aligned(x, 16) || !aligned(w13_prep, 16) || !aligned(a2, 2))
    return gemm_fail_shape(W, d, 2 * d->I, d->H, 0);
  nvfp4::GemmArgs a = gemm_args(d);
  a.offsets = expert_offsets;
  a.sorted_pair = sorted_pair;
  a.plan = plan;
  a.a_h = x;
  a.w_prep = w13_prep;
  a.g_w = gw13;
  a.out_h = a2;
  a.part = part;
  return launched(nvfp4::launch_gemm1(a, false, S(stream)), W);
}

int grouped_gemm1_swiglu_w4a16(const nvfp4_moe_dims* d, const uint16_t* x, const int32_t* sorted_pair,
                               const int32_t* expert_offsets, const int32_t* plan, const uint8_t* w13_prep,
                               const float* gw13, uint16_t* a2, void* stream) {
  return grouped_gemm1_swiglu_w4a16_impl("grouped_gemm1_swiglu_w4a16", nvfp4::kPartAll, d, x, sorted_pair,
                                         expert_offsets, plan, w13_prep, gw13, a2, stream);
}

int grouped_gemm1_swiglu_w4a16_part(const nvfp4_moe_dims* d, const uint16_t* x, const int32_t* sorted_pair,
                                    const int32_t* expert_offsets, const int32_t* plan,
                                    const uint8_t* w13_prep, const float* gw13, uint16_t* a2, int part,
                                    void* stream) {
  if (part < 0 || part > 2)
    return fail(NVFP4_EINVAL, "%s: EINVAL part=%d (0..2)", "grouped_gemm1_swiglu_w4a16_part", part);
  return grouped_gemm1_swiglu_w4a16_impl("grouped_gemm1_swiglu_w4a16_part", part, d, x, sorted_pair,
                                         expert_offsets, plan, w13_prep, gw13, a2, stream);
}

static int gemm2_common(const char* W, const nvfp4_moe_dims* d, const int32_t* expert_offsets,
                        const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                        const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype,
                        void* ws, size_t ws_bytes, bool need_gw = true) {
  if (int r = check_dims(d, W)) return r;
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_F32)
    return fail(NVFP4_EINVAL, "%s: EINVAL out_dtype=%d", W, out_dtype);
  const size_t need = grouped_gemm_workspace_size(d);
  if (d->T == 0) return NVFP4_OK;
  if (ws_bytes < need || !ws)
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld N=%d K=%d workspace_size=%zu "
                "needed=%zu", W, d->E + d->shared, (long long)pairs(d), d->H, d->I, ws_bytes, need);
  if (!expert_offsets || !inv_pos || !plan || !topk_w || !w2_prep || (need_gw && !gw2) || !out ||
      !aligned(w2_prep, 16) || !aligned(ws, 16) || !aligned(out, out_dtype == NVFP4_F32 ? 16 : 8))
    return gemm_fail_shape(W, d, d->H, d->I, ws_bytes);
  return NVFP4_OK;
}

static int grouped_gemm2_combine_impl(const char* W, int part, const nvfp4_moe_dims* d, const uint8_t* a2_q,
                                      const uint8_t* a2_sf, const uint16_t* a2_deq, const float* g2,
                                      const int32_t* expert_offsets, const int32_t* inv_pos,
                                      const int32_t* plan, const float* topk_w, const uint8_t* w2_prep,
                                      const float* gw2, void* out, int out_dtype, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (int r = gemm2_common(W, d, expert_offsets, inv_pos, plan, topk_w, w2_prep, gw2, out,
                           out_dtype, ws, ws_bytes))
    return r;
  if (d->T == 0) return ok();
  if ((!a2_deq && (!a2_q || !a2_sf)) || !g2 || !aligned(a2_q, 16) || !aligned(a2_sf, 2) ||
      !aligned(a2_deq, 16))
    return gemm_fail_shape(W, d, d->H, d->I, ws_bytes);
  nvfp4::GemmArgs a = gemm_args(d);
  a.offsets = expert_offsets;
  a.inv_pos = inv_pos;
  a.plan = plan;
  a.topk_w = topk_w;
  a.a_q = a2_q;
  a.a_sf = a2_sf;
  a.a_h = a2_deq;
  a.g_a = g2;
  a.w_prep = w2_prep;
  a.g_w = gw2;
  a.d_ws = static_cast<float*>(ws);
  a.out = out;
  a.out_dtype = out_dtype;
  a.part = part;
  return launched(nvfp4::launch_gemm2_combine(a, true, S(stream)), W);
}

int grouped_gemm2_combine(const nvfp4_moe_dims* d, const uint8_t* a2_q, const uint8_t* a2_sf,
                          const uint16_t* a2_deq, const float* g2, const int32_t* expert_offsets,
                          const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                          const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype, void* ws,
                          size_t ws_bytes, void* stream) {
  return grouped_gemm2_combine_impl("grouped_gemm2_combine", nvfp4::kPartAll, d, a2_q, a2_sf, a2_deq, g2,
                                    expert_offsets, inv_pos, plan, topk_w, w2_prep, gw2, out, out_dtype, ws,
                                    ws_bytes, stream);
}

int grouped_gemm2_combine_part(const nvfp4_moe_dims* d, const uint8_t* a2_q, const uint8_t* a2_sf,
                               const uint16_t* a2_deq, const float* g2, const int32_t* expert_offsets,
                               const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                               const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype, void* ws,
                               size_t ws_bytes, int part, void* stream) {
  if (part < 0 || part > 3)
    return fail(NVFP4_EINVAL, "%s: EINVAL part=%d (0..3)", "grouped_gemm2_combine_part", part);
  return grouped_gemm2_combine_impl("grouped_gemm2_combine_part", part, d, a2_q, a2_sf, a2_deq, g2,
                                    expert_offsets, inv_pos, plan, topk_w, w2_prep, gw2, out, out_dtype, ws,
                                    ws_bytes, stream);
}

static int grouped_gemm2_combine_w4a16_impl(const char* W, int part, const nvfp4_moe_dims* d,
                                            const uint16_t* a2, const int32_t* expert_offsets,
                                            const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                                            const uint8_t* w2_prep, const float* gw2, void* out,
                                            int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (int r = gemm2_common(W, d, expert_offsets, inv_pos, plan, topk_w, w2_prep, gw2, out,
                           out_dtype, ws, ws_bytes))
    return r;
  if (d->T == 0) return ok();
  if (!a2 || !aligned(a2, 16)) return gemm_fail_shape(W, d, d->H, d->I, ws_bytes);
  nvfp4::GemmArgs a = gemm_args(d);
  a.offsets = expert_offsets;
  a.inv_pos = inv_pos;
  a.plan = plan;
  a.topk_w = topk_w;
  a.a_h = a2;
  a.w_prep = w2_prep;
  a.g_w = gw2;
  a.d_ws = static_cast<float*>(ws);
  a.out = out;
  a.out_dtype = out_dtype;
  a.part = part;
  return launched(nvfp4::launch_gemm2_combine(a, false, S(stream)), W);
}

int grouped_gemm2_combine_w4a16(const nvfp4_moe_dims* d, const uint16_t* a2, const int32_t* expert_offsets,
                                const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                                const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype, void* ws,
                                size_t ws_bytes, void* stream) {
  return grouped_gemm2_combine_w4a16_impl("grouped_gemm2_combine_w4a16", nvfp4::kPartAll, d, a2,
                                          expert_offsets, inv_pos, plan, topk_w, w2_prep, gw2, out, out_dtype,
                                          ws, ws_bytes, stream);
}

int grouped_gemm2_combine_w4a16_part(const nvfp4_moe_dims* d, const uint16_t* a2,
                                     const int32_t* expert_offsets, const int32_t* inv_pos,
                                     const int32_t* plan, const float* topk_w, const uint8_t* w2_prep,
                                     const float* gw2, void* out, int out_dtype, void* ws, size_t ws_bytes,
                                     int part, void* stream) {
  if (part < 0 || part > 3)
    return fail(NVFP4_EINVAL, "%s: EINVAL part=%d (0..3)", "grouped_gemm2_combine_w4a16_part", part);
  return grouped_gemm2_combine_w4a16_impl("grouped_gemm2_combine_w4a16_part", part, d, a2, expert_offsets,
                                          inv_pos, plan, topk_w, w2_prep, gw2, out, out_dtype, ws, ws_bytes,
                                          stream);
}

// ------------------------------------------------------------------ MXFP4 layer
size_t mxfp4_prep_expert_weights_size(const nvfp4_moe_dims* d, int which) {
  if (check_dims(d, "mxfp4_prep_expert_weights_size") || (which != 13 && which != 2)) return 0;
  const int64_t slots = d->E + d->shared;
  return which == 13 ? nvfp4::mx_expert_prep_bytes(slots, 2 * (int64_t)d->I, d->H)
                     : nvfp4::mx_expert_prep_bytes(slots, d->H, d->I);
}

int mxfp4_prep_expert_weights(const nvfp4_moe_dims* d, int which, const uint8_t* q, const uint8_t* ex,
                              uint8_t* prep, void* stream) {
  const char* W = "mxfp4_prep_expert_weights";
  if (int r = check_dims(d, W)) return r;
  if (which != 13 && which != 2) return fail(NVFP4_EINVAL, "%s: EINVAL which=%d (13 or 2)", W, which);
  if (!q || !ex || !prep) return fail(NVFP4_EINVAL, "%s: EINVAL null pointer", W);
  if (!aligned(q, 16) || !aligned(prep, 16))
    return fail(NVFP4_EINVAL, "%s: EINVAL q and prep must be 16-byte aligned", W);
  const int64_t slots = d->E + d->shared;
  const int64_t N = which == 13 ? 2 * (int64_t)d->I : d->H;
  const int64_t K = which == 13 ? d->H : d->I;
  return launched(nvfp4::launch_mx_expert_prep(slots, N, K, which == 13 ? d->I : 0, q, ex, prep, S(stream)), W);
}

namespace {
nvfp4::MxGemmArgs mx_args(const nvfp4_moe_dims* d) {
  nvfp4::MxGemmArgs a{};
  a.T = d->T;
  a.topk = d->topk;
  a.E = d->E;
  a.shared = d->shared;
  a.H = d->H;
  a.I = d->I;
  return a;
}
// Byte offsets of the activation operands travel as 32-bit values.
bool mx_offsets_fit(const nvfp4_moe_dims* d) {
  const int64_t P = pairs(d);
  return (int64_t)d->T * d->H / 2 < (int64_t(1) << 31) && P * d->I / 2 < (int64_t(1) << 31) &&
         (int64_t)2 * d->I * d->H / 2 < (int64_t(1) << 31);
}
}  // namespace

static int grouped_gemm1_swiglu_mxfp4_impl(const char* W, int part, const nvfp4_moe_dims* d,
                                           const uint8_t* a1_q, const uint8_t* a1_e,
                                           const int32_t* sorted_pair, const int32_t* expert_offsets,
                                           const int32_t* plan, const uint8_t* w13_prep, uint8_t* a2_q,
                                           uint8_t* a2_e, void* stream) {
  if (int r = check_dims(d, W)) return r;
  if (!mx_offsets_fit(d))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE num_experts=%d M=%lld N=%d K=%d (operand offsets must fit 31 bits)", W,
                d->E + d->shared, (long long)pairs(d), 2 * d->I, d->H);
  if (d->T == 0) return ok();
  if (!a1_q || !a1_e || !sorted_pair || !expert_offsets || !plan || !w13_prep || !a2_q || !a2_e ||
      !aligned(a1_q, 16) || !aligned(a1_e, 4) || !aligned(w13_prep, 16) || !aligned(a2_q, 16) ||
      !aligned(a2_e, 4))
    return gemm_fail_shape(W, d, 2 * d->I, d->H, 0);
  nvfp4::MxGemmArgs a = mx_args(d);
  a.sorted_pair = sorted_pair;
  a.plan = plan;
  a.a_q = a1_q;
  a.a_e = a1_e;
  a.w_prep = w13_prep;
  a.out_q = a2_q;
  a.out_e = a2_e;
  a.part = part;
  return launched(nvfp4::launch_mx_gemm1_swiglu(a, S(stream)), W);
}

int grouped_gemm1_swiglu_mxfp4(const nvfp4_moe_dims* d, const uint8_t* a1_q, const uint8_t* a1_e,
                               const int32_t* sorted_pair, const int32_t* expert_offsets, const int32_t* plan,
                               const uint8_t* w13_prep, uint8_t* a2_q, uint8_t* a2_e, void* stream) {
  return grouped_gemm1_swiglu_mxfp4_impl("grouped_gemm1_swiglu_mxfp4", nvfp4::kPartAll, d, a1_q, a1_e,
                                         sorted_pair, expert_offsets, plan, w13_prep, a2_q, a2_e, stream);
}

int grouped_gemm1_swiglu_mxfp4_part(const nvfp4_moe_dims* d, const uint8_t* a1_q, const uint8_t* a1_e,
                                    const int32_t* sorted_pair, const int32_t* expert_offsets,
                                    const int32_t* plan, const uint8_t* w13_prep, uint8_t* a2_q,
                                    uint8_t* a2_e, int part, void* stream) {
  if (part < 0 || part > 2)
    return fail(NVFP4_EINVAL, "%s: EINVAL part=%d (0..2)", "grouped_gemm1_swiglu_mxfp4_part", part);
  return grouped_gemm1_swiglu_mxfp4_impl("grouped_gemm1_swiglu_mxfp4_part", part, d, a1_q, a1_e, sorted_pair,
                                         expert_offsets, plan, w13_prep, a2_q, a2_e, stream);
}

static int grouped_gemm2_combine_mxfp4_impl(const char* W, int part, const nvfp4_moe_dims* d,
                                            const uint8_t* a2_q, const uint8_t* a2_e,
                                            const int32_t* expert_offsets, const int32_t* inv_pos,
                                            const int32_t* plan, const float* topk_w, const uint8_t* w2_prep,
                                            void* out, int out_dtype, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (int r = gemm2_common(W, d, expert_offsets, inv_pos, plan, topk_w, w2_prep, nullptr, out, out_dtype, ws,
                           ws_bytes, false))
    return r;
  if (!mx_offsets_fit(d))
    return fail(NVFP4_ESHAPE, "%s: ESHAPE num_experts=%d M=%lld N=%d K=%d (operand offsets must fit 31 bits)", W,
                d->E + d->shared, (long long)pairs(d), d->H, d->I);
  if (d->T == 0) return ok();
  if (!a2_q || !a2_e || !aligned(a2_q, 16) || !aligned(a2_e, 4)) return gemm_fail_shape(W, d, d->H, d->I, ws_bytes);
  nvfp4::MxGemmArgs a = mx_args(d);
  a.inv_pos = inv_pos;
  a.plan = plan;
  a.topk_w = topk_w;
  a.a_q = a2_q;
  a.a_e = a2_e;
  a.w_prep = w2_prep;
  a.d_ws = static_cast<float*>(ws);
  a.out = out;
  a.out_dtype = out_dtype;
  a.part = part;
  return launched(nvfp4::launch_mx_gemm2_combine(a, S(stream)), W);
}

int grouped_gemm2_combine_mxfp4(const nvfp4_moe_dims* d, const uint8_t* a2_q, const uint8_t* a2_e,
                                const int32_t* expert_offsets, const int32_t* inv_pos, const int32_t* plan,
                                const float* topk_w, const uint8_t* w2_prep, void* out, int out_dtype,
                                void* ws, size_t ws_bytes, void* stream) {
  return grouped_gemm2_combine_mxfp4_impl("grouped_gemm2_combine_mxfp4", nvfp4::kPartAll, d, a2_q, a2_e,
                                          expert_offsets, inv_pos, plan, topk_w, w2_prep, out, out_dtype, ws,
                                          ws_bytes, stream);
}

int grouped_gemm2_combine_mxfp4_part(const nvfp4_moe_dims* d, const uint8_t* a2_q, const uint8_t* a2_e,
                                     const int32_t* expert_offsets, const int32_t* inv_pos,
                                     const int32_t* plan, const float* topk_w, const uint8_t* w2_prep,
                                     void* out, int out_dtype, void* ws, size_t ws_bytes, int part,
                                     void* stream) {
  if (part < 0 || part > 3)
    return fail(NVFP4_EINVAL, "%s: EINVAL part=%d (0..3)", "grouped_gemm2_combine_mxfp4_part", part);
  return grouped_gemm2_combine_mxfp4_impl("grouped_gemm2_combine_mxfp4_part", part, d, a2_q, a2_e,
                                          expert_offsets, inv_pos, plan, topk_w, w2_prep, out, out_dtype, ws,
                                          ws_bytes, stream);
}

// ------------------------------------------------------------------ GEMM2 without allocation
namespace {
// Scratch of grouped_gemm2_combine_noalloc: the per-row FP32 down-projection
// outputs [P][H] that the combine reads, in a file-scope device array (every
// GPU the library runs on holds its own copy until the process ends).  In
// host code the array's name is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(48) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(const char* W, float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NVFP4_ELAUNCH, "%s: ELAUNCH hipGetDevice: %s", W, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_EINVAL, "%s: EINVAL device %d beyond the %d supported", W, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(NVFP4_ELAUNCH, "%s: ELAUNCH hipGetSymbolAddress(scratch): %s", W, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}
}  // namespace

size_t grouped_gemm2_combine_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int grouped_gemm2_combine_noalloc(const nvfp4_moe_dims* d, const uint8_t* a2_q, const uint8_t* a2_sf,
                                  const uint16_t* a2_deq, const float* g2, const int32_t* expert_offsets,
                                  const int32_t* inv_pos, const int32_t* plan, const float* topk_w,
                                  const uint8_t* w2_prep, const float* gw2, void* out, int out_dtype,
                                  void* stream) {
  const char* W = "grouped_gemm2_combine_noalloc";
  if (int r = check_dims(d, W)) return r;
  const size_t need = grouped_gemm_workspace_size(d);
  if (need > kNoAllocScratchBytes)
    return fail(NVFP4_EWORKSPACE, "%s: EWORKSPACE num_experts=%d M=%lld N=%d K=%d needs %zu bytes of "
                "scratch; the static scratch holds %zu (P * H <= %zu)", W, d->E + d->shared,
                (long long)pairs(d), d->H, d->I, need, kNoAllocScratchBytes,
                kNoAllocScratchBytes / sizeof(float));
  if (d->T == 0) return ok();
  float* ws = nullptr;
  if (int r = scratch_of_current_device(W, &ws)) return r;
  const int r = grouped_gemm2_combine(d, a2_q, a2_sf, a2_deq, g2, expert_offsets, inv_pos, plan, topk_w,
                                      w2_prep, gw2, out, out_dtype, ws, kNoAllocScratchBytes, stream);
  if (r != NVFP4_OK) {
    // name this entry point in the message of the shared path
    std::string m = g_err;
    const std::string from = "grouped_gemm2_combine:";
    if (m.compare(0, from.size(), from) == 0) m = std::string(W) + ":" + m.substr(from.size());
    g_err = m;
  }
  return r;
}

}  // extern "C"
