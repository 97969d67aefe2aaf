// api.cpp -- the C ABI (include/qprefill.h): argument validation, launch,
// status reporting.  Every check runs before anything is enqueued, so an
// error leaves every output untouched; there is no CPU fallback ("Qwen3.5
// batched prefill has no f32 dequant for IQ2_XXS, IQ3_S, IQ3_XXS, Q2_K",
// sections "Cause" and title: an unsupported type is an InvalidParameter-style
// error and the engine fails closed).
#include <cmath>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "qprefill.h"
#include "qp_internal.h"

namespace {

thread_local char g_detail[512] = "";

qp_status fail(qp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return s;
}

qp_status ok() {
  g_detail[0] = '\0';
  return QP_OK;
}

qp_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool supported(int qtype) {
  return qtype == QP_F16W || qtype == QP_Q8_0 || qtype == QP_Q4_K || qtype == QP_Q5_K || qtype == QP_Q6_K ||
         qtype == QP_Q2_K;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every 32-bit index of the kernels in range

}  // namespace

extern "C" {

int64_t qp_block_size(int qtype) {
  switch (qtype) {
    case QP_F16W: return 1;
    case QP_Q8_0: case QP_Q4_0: return 32;
    case QP_Q4_K: case QP_Q5_K: case QP_Q6_K: case QP_Q2_K: return 256;
    default: return -1;
  }
}

int64_t qp_type_size(int qtype) {
  switch (qtype) {
    case QP_F16W: return 2;
    case QP_Q8_0: return 34;
    case QP_Q4_0: return 18;
    case QP_Q4_K: return 144;
    case QP_Q5_K: return 176;
    case QP_Q6_K: return 210;
    case QP_Q2_K: return 84;
    default: return -1;
  }
}

int64_t qp_row_bytes(int qtype, int64_t cols) {
  const int64_t qk = qp_block_size(qtype);
  if (qk < 0 || cols <= 0) return -1;
  return (cols + qk - 1) / qk * qp_type_size(qtype);
}

static qp_status dequant_common(int qtype, const void* src, int64_t rows, int64_t cols, void* dst, bool f16,
                                hipStream_t stream) {
  if (!supported(qtype)) return fail(QP_ERR_UNSUPPORTED_TYPE, "no dequant kernel for ggml type %d", qtype);
  if (rows < 0 || cols <= 0 || rows > kMaxDim || cols > kMaxDim)
    return fail(QP_ERR_INVALID_PARAMETER, "rows=%lld cols=%lld out of range", (long long)rows, (long long)cols);
  if (rows == 0) return ok();
  if (!src || !dst) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(src, 16)) return fail(QP_ERR_INVALID_PARAMETER, "src must be 16-byte aligned");
  if (!aligned(dst, f16 ? 2 : 4)) return fail(QP_ERR_INVALID_PARAMETER, "dst misaligned");
  if (rows * cols > ((int64_t)1 << 40)) return fail(QP_ERR_INVALID_PARAMETER, "tensor too large");
  return from_hip(qp::launch_dequant(qtype, f16, src, rows, cols, dst, stream), "dequant launch");
}

qp_status qp_dequant_f32(int qtype, const void* src, int64_t rows, int64_t cols, float* dst, hipStream_t stream) {
  return dequant_common(qtype, src, rows, cols, dst, false, stream);
}

qp_status qp_dequant_f16(int qtype, const void* src, int64_t rows, int64_t cols, uint16_t* dst,
                         hipStream_t stream) {
  return dequant_common(qtype, src, rows, cols, dst, true, stream);
}

static qp_status gemm_checks(int qtype, const void* w, int64_t n, int64_t k, const void* x, int64_t t, int64_t ldx,
                             size_t xsize, const float* y, int64_t ldy) {
  if (!supported(qtype)) return fail(QP_ERR_UNSUPPORTED_TYPE, "no prefill GEMM for ggml type %d", qtype);
  if (n <= 0 || k <= 0 || t < 0 || n > kMaxDim || k > kMaxDim || t > kMaxDim)
    return fail(QP_ERR_INVALID_PARAMETER, "n=%lld k=%lld t=%lld out of range", (long long)n, (long long)k,
                (long long)t);
  if (k % 256 != 0) return fail(QP_ERR_INVALID_PARAMETER, "k=%lld must be a multiple of 256", (long long)k);
  if (ldx < k || ldy < n) return fail(QP_ERR_INVALID_PARAMETER, "ldx < k or ldy < n");
  if ((ldx * (int64_t)xsize) % 16 != 0) return fail(QP_ERR_INVALID_PARAMETER, "ldx rows must be 16-byte multiples");
  if (t == 0) return ok();
  if (!w || !x || !y) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 16))
    return fail(QP_ERR_INVALID_PARAMETER, "w, x and y must be 16-byte aligned");
  return ok();
}

qp_status qp_prefill_gemm(int qtype, const void* w, int64_t n, int64_t k, const void* x, int x_dtype, int64_t t,
                          int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
  return qp_prefill_gemm_ws(qtype, w, n, k, x, x_dtype, t, ldx, y, ldy, nullptr, 0, stream);
}

qp_status qp_prefill_gemm_ws(int qtype, const void* w, int64_t n, int64_t k, const void* x, int x_dtype, int64_t t,
                             int64_t ldx, float* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (x_dtype != QP_F16 && x_dtype != QP_F32) return fail(QP_ERR_INVALID_PARAMETER, "x_dtype must be QP_F16 or QP_F32");
  qp_status st = gemm_checks(qtype, w, n, k, x, t, ldx, x_dtype == QP_F32 ? 4 : 2, y, ldy);
  if (st != QP_OK || t == 0) return st;
  if (workspace != nullptr) {
    if (!aligned(workspace, 16)) return fail(QP_ERR_INVALID_PARAMETER, "workspace must be 16-byte aligned");
    if (workspace_bytes < qp_prefill_gemm_workspace_bytes(n, k, t))
      return fail(QP_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu below the query", workspace_bytes);
  }
  return from_hip(qp::launch_gemm_split(qtype, w, n, k, x, x_dtype == QP_F32, t, ldx, y, ldy, (float*)workspace,
                                        (int64_t)(workspace_bytes / 4), stream),
                  "gemm launch");
}

qp_status qp_prefill_gemm_noalloc(int qtype, const void* w, int64_t n, int64_t k, const void* x, int x_dtype,
                                  int64_t t, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
  static_assert(QP_NOALLOC_SCRATCH_BYTES == qp::kNoAllocScratchBytes, "header states the scratch size");
  if (x_dtype != QP_F16 && x_dtype != QP_F32) return fail(QP_ERR_INVALID_PARAMETER, "x_dtype must be QP_F16 or QP_F32");
  qp_status st = gemm_checks(qtype, w, n, k, x, t, ldx, x_dtype == QP_F32 ? 4 : 2, y, ldy);
  if (st != QP_OK || t == 0) return st;
  const size_t need = qp_prefill_gemm_workspace_bytes(n, k, t);
  if (need > qp::kNoAllocScratchBytes)
    return fail(QP_ERR_WORKSPACE_TOO_SMALL, "this split needs %zu bytes of partial sums, above the %zu-byte static scratch",
                need, qp::kNoAllocScratchBytes);
  return from_hip(qp::launch_gemm_noalloc(qtype, w, n, k, x, x_dtype == QP_F32, t, ldx, y, ldy, stream),
                  "gemm_noalloc launch");
}

size_t qp_prefill_gemm_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  if (n <= 0 || k <= 0 || t < 0 || n > kMaxDim || k > kMaxDim || t > kMaxDim) return 0;
  const int parts = qp::gemm_ksplit_parts(n, k, t);
  int64_t floats = parts > 1 ? parts * t * n : 0;
  if (qp::wide_halves_shape(n, k, t) && t * n > floats) floats = t * n;  // the 256 x 256 tile's second K half
  return (size_t)((floats * 4 + 255) / 256 * 256);
}

qp_status qp_prefill_gemm_gate_up(int qtype, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                                  const uint16_t* x, int64_t t, int64_t ldx, float* y_gate, int64_t ldy_gate,
                                  float* y_up, int64_t ldy_up, hipStream_t stream) {
  qp_status st = gemm_checks(qtype, w_gate, n, k, x, t, ldx, 2, y_gate, ldy_gate);
  if (st != QP_OK) return st;
  st = gemm_checks(qtype, w_up, n, k, x, t, ldx, 2, y_up, ldy_up);
  if (st != QP_OK || t == 0) return st;
  return from_hip(qp::launch_gemm_gate_up(qtype, w_gate, w_up, n, k, x, t, ldx, y_gate, ldy_gate, y_up, ldy_up, stream),
                  "gemm_gate_up launch");
}

qp_status qp_prefill_gemm_qknorm(int qtype, const void* w, int64_t n, int64_t k, const uint16_t* x, int64_t t,
                                 int64_t ldx, int64_t head_dim, const float* gain, int64_t gain_head_stride,
                                 float eps, float* y, int64_t ldy, hipStream_t stream) {
  qp_status st = gemm_checks(qtype, w, n, k, x, t, ldx, 2, y, ldy);
  if (st != QP_OK) return st;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(QP_ERR_INVALID_PARAMETER, "head_dim=%lld must be 64, 128 or 256", (long long)head_dim);
  if (n % head_dim != 0) return fail(QP_ERR_INVALID_PARAMETER, "n must be a multiple of head_dim");
  if (!(eps > 0.f) || !isfinite(eps)) return fail(QP_ERR_INVALID_PARAMETER, "eps must be finite and > 0");
  if (gain_head_stride < 0) return fail(QP_ERR_INVALID_PARAMETER, "gain_head_stride must be >= 0");
  if (t == 0) return ok();
  if (!gain) return fail(QP_ERR_INVALID_PARAMETER, "null gain");
  return from_hip(qp::launch_gemm_qknorm(qtype, w, n, k, x, t, ldx, head_dim, gain, gain_head_stride, eps, y, ldy,
                                         stream),
                  "gemm_qknorm launch");
}

qp_status qp_prefill_gemm_qkv(int qtype, const void* w_q, int64_t n_q, const void* w_k, int64_t n_k,
                              const void* w_v, int64_t n_v, int64_t k, const uint16_t* x, int64_t t, int64_t ldx,
                              int64_t head_dim, const float* gain_q, int64_t gain_q_stride, const float* gain_k,
                              int64_t gain_k_stride, float eps, float* y_q, int64_t ldy_q, float* y_k, int64_t ldy_k,
                              float* y_v, int64_t ldy_v, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (n_v < 0) return fail(QP_ERR_INVALID_PARAMETER, "n_v=%lld must be >= 0", (long long)n_v);
  qp_status st = gemm_checks(qtype, w_q, n_q, k, x, t, ldx, 2, y_q, ldy_q);
  if (st != QP_OK) return st;
  st = gemm_checks(qtype, w_k, n_k, k, x, t, ldx, 2, y_k, ldy_k);
  if (st != QP_OK) return st;
  if (n_v > 0) {
    st = gemm_checks(qtype, w_v, n_v, k, x, t, ldx, 2, y_v, ldy_v);
    if (st != QP_OK) return st;
  }
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(QP_ERR_INVALID_PARAMETER, "head_dim=%lld must be 64, 128 or 256", (long long)head_dim);
  if (n_q % head_dim != 0 || n_k % head_dim != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "n_q and n_k must be multiples of head_dim");
  if (!(eps > 0.f) || !isfinite(eps)) return fail(QP_ERR_INVALID_PARAMETER, "eps must be finite and > 0");
  if (gain_q_stride < 0 || gain_k_stride < 0) return fail(QP_ERR_INVALID_PARAMETER, "gain strides must be >= 0");
  if (t == 0) return ok();
  if (!gain_q || !gain_k) return fail(QP_ERR_INVALID_PARAMETER, "null gain");
  const void* w[3] = {w_q, w_k, w_v};
  const int64_t n[3] = {n_q, n_k, n_v};
  const float* gain[3] = {gain_q, gain_k, nullptr};
  const int64_t gstride[3] = {gain_q_stride, gain_k_stride, 0};
  float* y[3] = {y_q, y_k, y_v};
  const int64_t ldy[3] = {ldy_q, ldy_k, ldy_v};
  if (workspace != nullptr) {
    if (!aligned(workspace, 16)) return fail(QP_ERR_INVALID_PARAMETER, "workspace must be 16-byte aligned");
    if (workspace_bytes < qp_prefill_gemm_qkv_workspace_bytes(n_q, n_k, n_v, t))
      return fail(QP_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu below the query", workspace_bytes);
  }
  return from_hip(qp::launch_gemm_qkv(qtype, w, n, k, x, t, ldx, head_dim, gain, gstride, eps, y, ldy,
                                      (float*)workspace, stream),
                  "gemm_qkv launch");
}

size_t qp_prefill_gemm_qkv_workspace_bytes(int64_t n_q, int64_t n_k, int64_t n_v, int64_t t) {
  if (n_q < 0 || n_k < 0 || n_v < 0 || t < 0 || n_k > kMaxDim || n_v > kMaxDim || t > kMaxDim) return 0;
  const int64_t n[3] = {n_q, n_k, n_v};
  return (size_t)((qp::qkv_split_partial_floats(n, t) * 4 + 255) / 256 * 256);
}

qp_status qp_moe_route_topk(const float* logits, int64_t t, int64_t n_experts, int64_t top_k, int renorm,
                            int32_t* ids, float* weights, hipStream_t stream) {
  if (t < 0 || t > kMaxDim || n_experts < 1 || n_experts > 1024 || top_k < 1 || top_k > n_experts || top_k > 64)
    return fail(QP_ERR_INVALID_PARAMETER, "t=%lld n_experts=%lld top_k=%lld out of range", (long long)t,
                (long long)n_experts, (long long)top_k);
  if (t == 0) return ok();
  if (!logits || !ids || !weights) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4))
    return fail(QP_ERR_INVALID_PARAMETER, "misaligned pointer");
  return from_hip(qp::launch_route_topk(logits, t, n_experts, top_k, renorm, ids, weights, stream), "router launch");
}

size_t qp_grouped_expert_workspace_bytes(int64_t t, int64_t top_k, int64_t n_experts, int64_t hidden,
                                         int64_t inter) {
  qp::MoeWorkspace ws;
  if (!qp::moe_workspace_layout(t, top_k, n_experts, hidden, inter, ws)) return 0;
  return ws.total;
}

qp_status qp_grouped_expert_gemm(int qtype, const void* w_gate, const void* w_up, const void* w_down,
                                 int64_t n_experts, int64_t hidden, int64_t inter, const uint16_t* x, int64_t t,
                                 int64_t top_k, const int32_t* ids, const float* weights, float* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!supported(qtype)) return fail(QP_ERR_UNSUPPORTED_TYPE, "no grouped expert GEMM for ggml type %d", qtype);
  if (n_experts < 1 || n_experts > 1024 || top_k < 1 || top_k > n_experts || t < 0 || hidden <= 0 || inter <= 0)
    return fail(QP_ERR_INVALID_PARAMETER, "sizes out of range");
  if (hidden % 256 != 0 || inter % 256 != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "hidden and inter must be multiples of 256");
  if (hidden > kMaxDim || inter > kMaxDim || t * top_k > ((int64_t)1 << 31) - 1)
    return fail(QP_ERR_INVALID_PARAMETER, "sizes too large");
  qp::MoeWorkspace ws;
  qp::moe_workspace_layout(t, top_k, n_experts, hidden, inter, ws);
  if (t == 0) return ok();
  if (!w_gate || !w_up || !w_down || !x || !ids || !weights || !out || !workspace)
    return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(x, 16) || !aligned(out, 16) ||
      !aligned(ids, 4) || !aligned(weights, 4) || !aligned(workspace, 256))
    return fail(QP_ERR_INVALID_PARAMETER, "misaligned pointer");
  if (workspace_bytes < ws.total)
    return fail(QP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, ws.total);
  return from_hip(qp::launch_grouped_expert(qtype, w_gate, w_up, w_down, n_experts, hidden, inter, x, t, top_k, ids,
                                            weights, out, workspace, ws, stream),
                  "grouped expert launch");
}

qp_status qp_grouped_expert_dropped_pairs(const void* workspace, uint32_t* count, hipStream_t stream) {
  if (!workspace || !count) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(workspace, 256) || !aligned(count, 4)) return fail(QP_ERR_INVALID_PARAMETER, "misaligned pointer");
  return from_hip(hipMemcpyAsync(count, (const char*)workspace + QP_MOE_DROPPED_PAIRS_OFFSET, sizeof(uint32_t),
                                 hipMemcpyDefault, stream),
                  "dropped-pairs copy");
}

qp_status qp_rope(float* x, int64_t ldx, int64_t t, int64_t n_head, int64_t head_dim, int64_t pos0, double base,
                  hipStream_t stream) {
  if (t < 0 || t > kMaxDim || n_head < 1 || n_head > 4096 || head_dim < 2 || head_dim > 1024 || head_dim % 2 != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "t=%lld n_head=%lld head_dim=%lld out of range", (long long)t,
                (long long)n_head, (long long)head_dim);
  if (ldx < n_head * head_dim) return fail(QP_ERR_INVALID_PARAMETER, "ldx=%lld below n_head * head_dim", (long long)ldx);
  if (pos0 < 0 || pos0 > ((int64_t)1 << 40)) return fail(QP_ERR_INVALID_PARAMETER, "pos0=%lld", (long long)pos0);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(QP_ERR_INVALID_PARAMETER, "base must be finite and > 1");
  if (t == 0) return ok();
  if (!x) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(x, 4)) return fail(QP_ERR_INVALID_PARAMETER, "misaligned pointer");
  return from_hip(qp::launch_rope(x, ldx, t, n_head, head_dim, pos0, base, stream), "rope launch");
}

qp_status qp_kv_cache_write(int kv_type, const float* src, int64_t lds, int64_t t, int64_t n_kv_head,
                            int64_t head_dim, void* cache, int64_t row0, hipStream_t stream) {
  if (kv_type != QP_F16W && kv_type != QP_Q8_0 && kv_type != QP_Q4_0)
    return fail(QP_ERR_UNSUPPORTED_TYPE, "no KV cache rows of ggml type %d", kv_type);
  if (t < 0 || t > kMaxDim || n_kv_head < 1 || n_kv_head > 4096 || head_dim < 32 || head_dim > 1024 ||
      head_dim % 32 != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "t=%lld n_kv_head=%lld head_dim=%lld out of range", (long long)t,
                (long long)n_kv_head, (long long)head_dim);
  if (lds < n_kv_head * head_dim || lds % 4 != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "lds=%lld: at least n_kv_head * head_dim and a multiple of 4",
                (long long)lds);
  if (row0 < 0 || row0 + t > kMaxDim) return fail(QP_ERR_INVALID_PARAMETER, "row0=%lld out of range", (long long)row0);
  if (t == 0) return ok();
  if (!src || !cache) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  if (!aligned(src, 16) || !aligned(cache, kv_type == QP_F16W ? 4 : 2))
    return fail(QP_ERR_INVALID_PARAMETER, "misaligned pointer");
  return from_hip(qp::launch_kv_write(kv_type, src, lds, t, n_kv_head, head_dim, cache, row0, stream),
                  "kv write launch");
}

size_t qp_prompt_attention_workspace_bytes(int kv_type, int64_t kv_len, int64_t n_kv_head, int64_t head_dim) {
  if ((kv_type != QP_Q8_0 && kv_type != QP_Q4_0) || head_dim != 128 || kv_len <= 0 || kv_len >= ((int64_t)1 << 31) ||
      n_kv_head < 1 || n_kv_head > 1024)
    return 0;
  const int64_t one = kv_len * n_kv_head * head_dim * 2;  // binary16 rows of one cache
  return (size_t)(2 * ((one + 255) / 256 * 256));
}

static qp_status attention_impl(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                                int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv_head, int64_t head_dim,
                                float scale, float* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (kv_type != QP_F16W && kv_type != QP_Q8_0 && kv_type != QP_Q4_0)
    return fail(QP_ERR_UNSUPPORTED_TYPE, "no prompt attention over a KV cache of ggml type %d", kv_type);
  if (head_dim != 128) return fail(QP_ERR_INVALID_PARAMETER, "head_dim %lld (only 128)", (long long)head_dim);
  if (n_head < 1 || n_head > 1024 || n_kv_head < 1 || n_head % n_kv_head != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "n_head=%lld n_kv_head=%lld", (long long)n_head, (long long)n_kv_head);
  if (t < 0 || n_past < 0 || n_past + t > ((int64_t)1 << 31) - 1 - 256)
    return fail(QP_ERR_INVALID_PARAMETER, "n_past=%lld t=%lld out of range", (long long)n_past, (long long)t);
  if (((t + 127) / 128) * n_head > ((int64_t)1 << 24) - 1)  // 256-thread workgroups: under 2^32 threads
    return fail(QP_ERR_INVALID_PARAMETER, "t=%lld with %lld heads: grid too large", (long long)t, (long long)n_head);
  const int64_t width = n_head * head_dim;
  if (ldq < width || ldo < width || ldq % 4 != 0 || ldo % 4 != 0)
    return fail(QP_ERR_INVALID_PARAMETER, "ldq=%lld ldo=%lld for %lld columns", (long long)ldq, (long long)ldo,
                (long long)width);
  if (!std::isfinite(scale)) return fail(QP_ERR_INVALID_PARAMETER, "scale is not finite");
  if (scale == 0.0f) scale = (float)(1.0 / std::sqrt((double)head_dim));
  if (t == 0) return ok();
  if (!q || !k_cache || !v_cache || !out) return fail(QP_ERR_INVALID_PARAMETER, "null pointer");
  const size_t cache_align = kv_type == QP_F16W ? 16 : 2;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, cache_align) || !aligned(v_cache, cache_align))
    return fail(QP_ERR_INVALID_PARAMETER, "misaligned pointer");
  if (workspace != nullptr && kv_type != QP_F16W) {
    // decode both caches once into binary16 rows, then attend over those
    const int64_t kv_len = n_past + t;
    const size_t need = qp_prompt_attention_workspace_bytes(kv_type, kv_len, n_kv_head, head_dim);
    if (workspace_bytes < need)
      return fail(QP_ERR_WORKSPACE_TOO_SMALL, "attention workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(QP_ERR_INVALID_PARAMETER, "misaligned workspace");
    if (2 * kv_len * n_kv_head * (head_dim / 8) > ((int64_t)1 << 32) - 256)  // one thread per 8 values, K and V
      return fail(QP_ERR_INVALID_PARAMETER, "a cache of %lld rows is too large for one decode launch",
                  (long long)(kv_len * n_kv_head));
    uint8_t* kf = (uint8_t*)workspace;
    uint8_t* vf = kf + need / 2;
    hipError_t e = qp::launch_kv_decode_f16(kv_type, k_cache, v_cache, kv_len * n_kv_head, kf, vf, stream);
    if (e == hipSuccess)
      e = qp::launch_attention(QP_F16W, q, ldq, kf, vf, n_past, t, n_head, n_kv_head, scale, out, ldo, stream);
    return from_hip(e, "attention launch");
  }
  return from_hip(qp::launch_attention(kv_type, q, ldq, k_cache, v_cache, n_past, t, n_head, n_kv_head, scale, out,
                                       ldo, stream),
                  "attention launch");
}

qp_status qp_prompt_attention(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                              int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv_head, int64_t head_dim,
                              float scale, float* out, int64_t ldo, hipStream_t stream) {
  return attention_impl(kv_type, q, ldq, k_cache, v_cache, n_past, t, n_head, n_kv_head, head_dim, scale, out, ldo,
                        nullptr, 0, stream);
}

qp_status qp_prompt_attention_ws(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                                 int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv_head, int64_t head_dim,
                                 float scale, float* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return attention_impl(kv_type, q, ldq, k_cache, v_cache, n_past, t, n_head, n_kv_head, head_dim, scale, out, ldo,
                        workspace, workspace_bytes, stream);
}

const char* qp_status_string(qp_status s) {
  switch (s) {
    case QP_OK: return "QP_OK";
    case QP_ERR_INVALID_PARAMETER: return "QP_ERR_INVALID_PARAMETER";
    case QP_ERR_UNSUPPORTED_TYPE: return "QP_ERR_UNSUPPORTED_TYPE";
    case QP_ERR_WORKSPACE_TOO_SMALL: return "QP_ERR_WORKSPACE_TOO_SMALL";
    case QP_ERR_DEVICE: return "QP_ERR_DEVICE";
    default: return "QP_ERR_UNKNOWN";
  }
}

const char* qp_last_error_detail(void) { return g_detail; }

}  // extern "C"
