// qp_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qp {

hipError_t launch_dequant(int qtype, bool f16out, const void* src, int64_t rows, int64_t cols, void* dst,
                          hipStream_t s);

hipError_t launch_gemm(int qtype, const void* w, int64_t n, int64_t k, const void* x, bool x_f32, int64_t t,
                       int64_t ldx, float* y, int64_t ldy, hipStream_t s);
// The same with room for partial sums (partial_floats floats, 16-byte
// aligned; null: none): an under-filled 128-tile launch is split into
// gemm_ksplit_parts() K parts whose sums one pass adds in order.
hipError_t launch_gemm_split(int qtype, const void* w, int64_t n, int64_t k, const void* x, bool x_f32, int64_t t,
                             int64_t ldx, float* y, int64_t ldy, float* partial, int64_t partial_floats,
                             hipStream_t s);
int gemm_ksplit_parts(int64_t n, int64_t k, int64_t t);
bool wide_halves_shape(int64_t n, int64_t k, int64_t t);
// launch_gemm_split with the library's static device scratch as the room for
// partial sums (kNoAllocScratchBytes; no allocation, no caller workspace).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t launch_gemm_noalloc(int qtype, const void* w, int64_t n, int64_t k, const void* x, bool x_f32, int64_t t,
                               int64_t ldx, float* y, int64_t ldy, hipStream_t s);

hipError_t launch_gemm_qknorm(int qtype, const void* w, int64_t n, int64_t k, const uint16_t* x, int64_t t,
                              int64_t ldx, int64_t head_dim, const float* gain, int64_t gain_head_stride,
                              float eps, float* y, int64_t ldy, hipStream_t s);

// gate and up projections of one X (same n and k)
hipError_t launch_gemm_gate_up(int qtype, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                               const uint16_t* x, int64_t t, int64_t ldx, float* y_gate, int64_t ldy_gate, float* y_up,
                               int64_t ldy_up, hipStream_t s);

// q, k (per-head RMSNorm) and v (plain) projections of one X; n[i] == 0 skips
// one.  partial: room for qkv_split_partial_floats() floats that lets k and v
// run as two K halves (null: never split).
hipError_t launch_gemm_qkv(int qtype, const void* const w[3], const int64_t n[3], int64_t k, const uint16_t* x,
                           int64_t t, int64_t ldx, int64_t head_dim, const float* const gain[3],
                           const int64_t gstride[3], float eps, float* const y[3], const int64_t ldy[3],
                           float* partial, hipStream_t s);
int64_t qkv_split_partial_floats(const int64_t n[3], int64_t t);

hipError_t launch_route_topk(const float* logits, int64_t t, int64_t e, int64_t top_k, int renorm, int32_t* ids,
                             float* weights, hipStream_t s);

// Workspace carve-up of the grouped expert GEMM (offsets in bytes, each
// 256-byte aligned).
struct MoeWorkspace {
  size_t header, ccount, cbad, cpref, counts, offsets, ntiles, tiles, ntiles2, tiles2, list, rowmax, hbuf, ubuf, h16,
      dbuf, total;
  int64_t max_tiles, max_tiles2, nchunks;
};
bool moe_workspace_layout(int64_t t, int64_t top_k, int64_t n_experts, int64_t hidden, int64_t inter,
                          MoeWorkspace& ws);

hipError_t launch_grouped_expert(int qtype, const void* w_gate, const void* w_up, const void* w_down,
                                 int64_t n_experts, int64_t hidden, int64_t inter, const uint16_t* x, int64_t t,
                                 int64_t top_k, const int32_t* ids, const float* weights, float* out,
                                 void* workspace, const MoeWorkspace& ws, hipStream_t s);

// Rotary step in place (half-split pairs) and the write of K / V rows into a
// binary16, Q8_0 or Q4_0 KV cache at cache rows (row0 + i) * n_kv + g.
hipError_t launch_rope(float* x, int64_t ldx, int64_t t, int64_t n_head, int64_t head_dim, int64_t pos0, double base,
                       hipStream_t s);
hipError_t launch_kv_write(int kv_type, const float* src, int64_t lds, int64_t t, int64_t n_kv, int64_t head_dim,
                           void* cache, int64_t row0, hipStream_t s);

// Causal prompt attention over a binary16 or Q8_0 KV cache, head_dim 128.
int64_t attention_row_bytes(int kv_type);
// The rows of a Q8_0 or Q4_0 K and V cache (head_dim 128) as binary16 rows,
// the values the attention kernel stages from them; one launch.
hipError_t launch_kv_decode_f16(int kv_type, const void* k_src, const void* v_src, int64_t rows, void* k_dst,
                                void* v_dst, hipStream_t s);
hipError_t launch_attention(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                            int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv, float scale, float* out,
                            int64_t ldo, hipStream_t s);

// geometry of the GEMM tiles (the MoE layout and the ABI checks use them)
constexpr int kTileM = 128;
constexpr int kTileN = 128;

}  // namespace qp
