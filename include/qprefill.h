/*
 * qprefill.h -- C ABI of the MI355X (gfx950) quantized prefill library.
 *
 * The operation: the batched prefill of a GGUF-quantized transformer runs a
 * chunk of T prompt tokens through each projection as one product
 * Y[T x N] = X[T x K] . W^T, where W (N output rows of K input weights) is
 * held in a block-quantized GGUF type and is dequantized on the way in.
 *   - "QK-norm models take the FP16 batched prefill" (aprender PR), "What
 *     changes": chunked batched prefill in FP16 for models with a per-head
 *     QK norm (FP8 fails parity on them).
 *   - "Qwen3.5 batched prefill has no f32 dequant for IQ2_XXS, IQ3_S,
 *     IQ3_XXS, Q2_K" (aprender issue), "Cause": every projection weight is
 *     dequantized to f32 before the GEMM and the f16 copy is built from that
 *     f32 value; an unsupported type is an InvalidParameter error, and the
 *     engine fails closed instead of falling back to the CPU.  "Acceptance
 *     (each row)": the dequant is bit-exact with the CPU oracle, including a
 *     partial last block, and writes nothing outside its output.
 *   - "CUDA prefill VRAM loans and SM75 Q4/native-IQ opt-ins" (Strata PR),
 *     "Summary" and "Correctness and safety": the routed experts get a fused
 *     prefill path that picks the same experts for each token, weighs them
 *     the same and adds their outputs up in the same order as the unfused
 *     path does.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are device memory of the current HIP device;
 *     (host) are host memory.  The caller owns every buffer.  The library
 *     never allocates, frees or synchronizes; the caller-supplied workspace
 *     is the only scratch memory, except for qp_prefill_gemm_noalloc, whose
 *     partial sums go to a fixed static device array of the library.
 *   - Work is enqueued on `stream` (NULL = the null stream) and is
 *     asynchronous: a QP_OK return means "validated and launched".
 *   - Arguments are validated before anything is launched.  On any error
 *     nothing is launched and no output is written.  There is no CPU
 *     fallback for any operation.
 *   - Block layouts (GGUF / ggml on-disk convention, little-endian fp16):
 *       F16    2 B per weight      : the weight as binary16 (ggml type 1);  w = that value
 *       Q8_0  34 B per 32 weights  : d f16 @0, qs int8[32] @2;  w = d*q
 *       Q4_K 144 B per 256 weights : d f16 @0, dmin f16 @2, 12 bytes of packed
 *                                    6-bit (scale, min) for 8 sub-blocks of 32 @4,
 *                                    qs u8[128] (4-bit quants) @16;  w = d*sc*q - dmin*m
 *       Q5_K 176 B per 256 weights : d f16 @0, dmin f16 @2, the Q4_K scale bytes @4,
 *                                    qh u8[32] @16, qs u8[128] @48; q (5 bits) = the
 *                                    Q4_K nibble of qs | bit (i/32) of qh[i%32] << 4;
 *                                    w = d*sc*q - dmin*m
 *       Q6_K 210 B per 256 weights : ql u8[128] @0, qh u8[64] @128, scales int8[16] @192,
 *                                    d f16 @208;  w = d*sc*(q - 32), q 6 bits
 *       Q2_K  84 B per 256 weights : scales u8[16] (4-bit scale | 4-bit min << 4) @0,
 *                                    qs u8[64] (2-bit quants) @16, d f16 @80, dmin f16 @82;
 *                                    w = d*sc*q - dmin*m
 *     A weight tensor of R rows x C columns is R rows of ceil(C/QK) whole
 *     blocks, back to back (row stride = qp_row_bytes(qtype, C)).
 *   - Type ids are the ggml type numbers.
 */
#ifndef QPREFILL_H
#define QPREFILL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QP_OK = 0,
  QP_ERR_INVALID_PARAMETER = 1,   /* bad size, stride, alignment, pointer or option */
  QP_ERR_UNSUPPORTED_TYPE = 2,    /* qtype is not F16, Q8_0, Q4_K, Q5_K, Q6_K or Q2_K */
  QP_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the size query */
  QP_ERR_DEVICE = 4               /* the HIP runtime reported an error at launch */
} qp_status;

typedef enum { QP_F16W = 1, QP_Q4_0 = 2, QP_Q8_0 = 8, QP_Q2_K = 10, QP_Q4_K = 12, QP_Q5_K = 13, QP_Q6_K = 14 } qp_qtype;

typedef enum { QP_F32 = 0, QP_F16 = 1 } qp_dtype;

/* Weights per block of a GGUF block type ("Qwen3.5 batched prefill has no f32
 * dequant ...", "Cause": the dequant covers the model's block types): 1
 * (F16), 32 (Q8_0, Q4_0) or 256 (K types); -1 for an unsupported type. */
int64_t qp_block_size(int qtype);

/* Bytes per block (same passage): 2, 34 (Q8_0), 18 (Q4_0), 144, 176, 210,
 * 84; -1 for an unsupported type. */
int64_t qp_type_size(int qtype);

/* Bytes of one row of `cols` weights (same passage; a row ends in a partial
 * block when cols % QK != 0, "Acceptance (each row)"): ceil(cols / QK) *
 * type_size.  -1 for an unsupported type or cols <= 0. */
int64_t qp_row_bytes(int qtype, int64_t cols);

/*
 * Dequantize a rows x cols tensor to f32 ("Cause": the f32 dequant of every
 * projection weight; "Acceptance (each row)": bit-exact, partial last block).
 *   src (device): rows * qp_row_bytes(qtype, cols) bytes, 16-byte aligned.
 *   dst (device): rows * cols floats, dense row-major: element (r, c) at
 *                 dst[r * cols + c]; 4-byte aligned.  Only these elements
 *                 are written: the unused quants of a partial last block are
 *                 ignored.
 * Values are computed in binary32, left to right, nearest-even:
 *   F16 the value itself;  Q8_0 d*q;  Q4_K, Q5_K, Q2_K (d*sc)*q - dmin*m;  Q6_K (d*sc)*(q-32).
 * rows == 0 is a no-op.  Errors: QP_ERR_UNSUPPORTED_TYPE, or
 * QP_ERR_INVALID_PARAMETER for rows < 0, cols <= 0, a NULL or misaligned
 * pointer.
 */
qp_status qp_dequant_f32(int qtype, const void* src, int64_t rows, int64_t cols, float* dst,
                         hipStream_t stream);

/*
 * Same as qp_dequant_f32, but each value is the binary16 (nearest-even,
 * subnormals kept, overflow to +-inf) of the f32 dequant ("Cause": the f16
 * copy is built from the f32 dequant).  dst (device): rows * cols binary16
 * bit patterns, 2-byte aligned.
 */
qp_status qp_dequant_f16(int qtype, const void* src, int64_t rows, int64_t cols, uint16_t* dst,
                         hipStream_t stream);

/*
 * Prefill projection ("What changes": batched prefill of a chunk of prompt
 * tokens in FP16):  y[t*ldy + n] = sum_k x[t*ldx + k] * W[n, k]
 *   w (device): the N x K weight tensor in `qtype`, 16-byte aligned.
 *   x (device): T x K activations, row stride ldx elements, binary16
 *               (x_dtype QP_F16) or f32 (QP_F32, rounded to binary16 on
 *               load); 16-byte aligned with ldx * element size a multiple
 *               of 16 bytes.
 *   y (device): T x N f32 outputs, row stride ldy (>= n); 16-byte aligned.
 * W is dequantized on load (nearest-even binary16 of the exact f32 value)
 * and never stored; products run on FP16 MFMA with f32 accumulation.
 * Requires k % 256 == 0.  t == 0 is a no-op.
 * Errors: QP_ERR_UNSUPPORTED_TYPE; QP_ERR_INVALID_PARAMETER for sizes or
 * strides out of range or misaligned pointers.
 */
qp_status qp_prefill_gemm(int qtype, const void* w, int64_t n, int64_t k, const void* x, int x_dtype,
                          int64_t t, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

/*
 * qp_prefill_gemm with an optional workspace, so that a launch whose shape
 * would leave the GPU under-filled can use all of it (a shape-dependent
 * choice of work split, as the per-format shape probe of "CUDA prefill VRAM
 * loans and SM75 Q4/native-IQ opt-ins", section "Summary", makes one per
 * weight format):
 *   workspace (device): qp_prefill_gemm_workspace_bytes(n, k, t) bytes,
 *     16-byte aligned, no initial contents needed; NULL (or a query of 0):
 *     exactly qp_prefill_gemm.
 * Where the 128-token tile's launch has fewer tiles than the GPU has compute
 * units, K is split into 2, 4 or 8 parts of whole 256-weight blocks; each
 * part writes its partial sums into the workspace and one more pass adds
 * them in part order into y.  Likewise, for Q2_K weights, K >= 8192 and
 * exactly half a round of 256 x 256 tiles, the two K halves run in one
 * launch of that tile, the second half's sums go to the workspace and one
 * pass adds them into y.  The result is the same on every call with the
 * same inputs and matches qp_prefill_gemm within the GEMM tolerance (the
 * summation order differs).  Calls that share a workspace must not run
 * concurrently.  Errors: those of qp_prefill_gemm, and
 * QP_ERR_WORKSPACE_TOO_SMALL for a non-NULL workspace below the query.
 */
qp_status qp_prefill_gemm_ws(int qtype, const void* w, int64_t n, int64_t k, const void* x, int x_dtype,
                             int64_t t, int64_t ldx, float* y, int64_t ldy, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Bytes of the workspace qp_prefill_gemm_ws may use for these sizes on the
 * current device, whatever the weight type (parts * t * n floats for the
 * 128-token split, t * n for the K halves, rounded up to 256); 0 when no
 * split applies, or for sizes out of range (the shape-dependent split of the
 * Strata PR's "Summary", as for qp_prefill_gemm_ws). */
size_t qp_prefill_gemm_workspace_bytes(int64_t n, int64_t k, int64_t t);

/*
 * qp_prefill_gemm_ws for callers that cannot allocate (code under HIP graph
 * capture, serving loops without an allocator, harnesses that forbid
 * hipMalloc): the same split and the same kernels, with the partial sums in a
 * static device array of QP_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  The caller passes inputs and
 * outputs only; the call allocates and frees nothing.  Results are bit for
 * bit those of qp_prefill_gemm_ws with a workspace.
 * On a GPU of up to 256 compute units every split fits the scratch; a split
 * that would need more (qp_prefill_gemm_workspace_bytes above
 * QP_NOALLOC_SCRATCH_BYTES) is rejected with QP_ERR_WORKSPACE_TOO_SMALL.
 * The first call on a device looks up that device's copy of the array.
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents (every partial sum is written before it is read, so nothing needs
 * clearing): calls that overlap on one GPU, on any streams, race.
 * Errors: those of qp_prefill_gemm_ws.
 */
#define QP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
qp_status qp_prefill_gemm_noalloc(int qtype, const void* w, int64_t n, int64_t k, const void* x, int x_dtype,
                                  int64_t t, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

/*
 * The two input projections of a feed-forward layer over one chunk ("What
 * changes": batched prefill of a chunk of prompt tokens in FP16, one product
 * per projection):
 *   y_gate = the qp_prefill_gemm result for (w_gate, n)
 *   y_up   = the qp_prefill_gemm result for (w_up, n)
 * over the same binary16 x (T x K, row stride ldx), with one qtype, n and k.
 * Where the two projections' tiles together fill the GPU this is a single
 * launch; otherwise it is the two calls.  Each output matches its separate
 * call within the GEMM tolerance (the summation order may differ), and every
 * call with the same inputs gives the same bits.  The outputs must not
 * overlap each other or x.  Requirements and errors are those of
 * qp_prefill_gemm with x_dtype QP_F16, for each projection.
 */
qp_status qp_prefill_gemm_gate_up(int qtype, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                                  const uint16_t* x, int64_t t, int64_t ldx, float* y_gate, int64_t ldy_gate,
                                  float* y_up, int64_t ldy_up, hipStream_t stream);

/*
 * Prefill projection with the per-head RMSNorm of QK-norm models fused into
 * the epilogue ("What changes": per-head QK norm):  with Y = X . W^T as in
 * qp_prefill_gemm, for each token t and head h (columns h*head_dim ..
 * h*head_dim + head_dim - 1):
 *   y[t, h*hd + j] = Y[t, h*hd + j] / sqrt(mean_j Y[t, h*hd + j]^2 + eps)
 *                    * gain[h * gain_head_stride + j]
 *   gain (device): f32; gain_head_stride 0 shares one head_dim vector
 *                  across heads, head_dim gives each head its own.
 *   x (device): binary16 activations (as qp_prefill_gemm with QP_F16).
 * Requires head_dim in {64, 128, 256}, n % head_dim == 0, finite eps > 0.
 * Heads of 64 and 128 columns are normalised in the projection's epilogue;
 * a head of 256 columns spans two output tiles, so the projection stores Y
 * and a second pass normalises each head of the stored rows in place (the
 * same arithmetic).
 */
qp_status qp_prefill_gemm_qknorm(int qtype, const void* w, int64_t n, int64_t k, const uint16_t* x,
                                 int64_t t, int64_t ldx, int64_t head_dim, const float* gain,
                                 int64_t gain_head_stride, float eps, float* y, int64_t ldy,
                                 hipStream_t stream);

/*
 * The attention-input projections of one chunk in one call ("What changes":
 * batched prefill of QK-norm models in FP16, the per-head RMSNorm on Q and K):
 *   y_q = the qp_prefill_gemm_qknorm result for (w_q, n_q, gain_q, gain_q_stride)
 *   y_k = the qp_prefill_gemm_qknorm result for (w_k, n_k, gain_k, gain_k_stride)
 *   y_v = the qp_prefill_gemm result for (w_v, n_v) with binary16 x
 * over the same x (T x K binary16, row stride ldx), with one qtype, k,
 * head_dim and eps.  When the three projections' output tiles together fill
 * the GPU and head_dim <= 128 this is a single launch (k and v alone often do
 * not fill it: 1024 outputs at T = 2048 make 64 tiles); otherwise it is the
 * three calls.  Results match
 * the separate calls within the GEMM tolerance (summation order may differ);
 * y_q matches its separate call bit for bit, and every call with the same
 * inputs gives the same bits.
 *   workspace (device, optional): qp_prefill_gemm_qkv_workspace_bytes(...)
 *     bytes, 16-byte aligned, no initial contents needed.  With it, where the
 *     single launch's last round of tiles would be only partly filled (and
 *     k % 512 == 0, n_k and n_v multiples of 8, ldy_k and ldy_v multiples of
 *     4), k and v each run as two K
 *     halves that write partial sums there; a second pass adds the halves in
 *     order and applies k's head norm.  NULL: no split.  Calls that share a
 *     workspace must not run concurrently.
 * n_v == 0 leaves v out (w_v, y_v unused).  The three outputs must not
 * overlap.  Requirements and errors are those of the two calls for each
 * projection, and QP_ERR_WORKSPACE_TOO_SMALL for a non-NULL workspace below
 * the query.
 */
qp_status qp_prefill_gemm_qkv(int qtype, const void* w_q, int64_t n_q, const void* w_k, int64_t n_k,
                              const void* w_v, int64_t n_v, int64_t k, const uint16_t* x, int64_t t, int64_t ldx,
                              int64_t head_dim, const float* gain_q, int64_t gain_q_stride, const float* gain_k,
                              int64_t gain_k_stride, float eps, float* y_q, int64_t ldy_q, float* y_k, int64_t ldy_k,
                              float* y_v, int64_t ldy_v, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Bytes of the optional workspace of qp_prefill_gemm_qkv (partial sums of k
 * and v: 2 * t * (n_k + n_v) floats, rounded up to 256; the work split of the
 * Strata PR's "Summary"); 0 for sizes out of range. */
size_t qp_prefill_gemm_qkv_workspace_bytes(int64_t n_q, int64_t n_k, int64_t n_v, int64_t t);

/*
 * Router of a routed-expert layer (Strata PR, "Correctness and safety": the
 * fused path must choose and weigh the experts exactly as the unfused one):
 * for each token t,
 * p = softmax(logits[t, :]) over n_experts; the top_k experts by logit,
 * largest first, ties to the lower expert index; weight = p of each chosen
 * expert (renorm != 0 divides the chosen weights by their sum).
 *   logits (device): t x n_experts f32.   ids (device): t x top_k int32.
 *   weights (device): t x top_k f32.
 * Requires 1 <= top_k <= min(n_experts, 64) and n_experts <= 1024.
 */
qp_status qp_moe_route_topk(const float* logits, int64_t t, int64_t n_experts, int64_t top_k,
                            int renorm, int32_t* ids, float* weights, hipStream_t stream);

/* Workspace bytes qp_grouped_expert_gemm needs for these sizes (0 on a bad
 * size): the token lists of the Strata PR's fused expert path ("Summary"),
 * the h rows between the passes and the per-pair outputs. */
size_t qp_grouped_expert_workspace_bytes(int64_t t, int64_t top_k, int64_t n_experts, int64_t hidden,
                                         int64_t inter);

/*
 * Routed expert FFN over per-expert token lists (Strata PR, "Summary": fused
 * routed-expert prefill; "Correctness and safety": the experts chosen, their
 * weights and the order of the sum stay those of the unfused path):  for
 * token t and slot s with expert e = ids[t, s]:
 *   g = x[t] . Wg_e^T, u = x[t] . Wu_e^T           (inter values each)
 *   h = SiLU(g) * u = g / (1 + exp(-g)) * u
 *   out[t, :] = sum over s = 0..top_k-1, in slot order, of weights[t, s] * (h . Wd_e^T)
 *   w_gate, w_up (device): n_experts tensors of inter x hidden in `qtype`,
 *                          back to back (expert stride inter * row_bytes(hidden)).
 *   w_down (device): n_experts tensors of hidden x inter (stride hidden * row_bytes(inter)).
 *   x (device): t x hidden binary16, row stride hidden.
 *   ids, weights (device): t x top_k int32 / f32.  A pair whose id is out of
 *                          [0, n_experts) contributes nothing and is counted
 *                          in the workspace header (the aprender issue's
 *                          "Cause": bad input is reported, never absorbed;
 *                          qp_grouped_expert_dropped_pairs reads the count).
 *   out (device): t x hidden f32, row stride hidden.
 *   workspace (device): >= qp_grouped_expert_workspace_bytes(...), 256-byte
 *                       aligned; its contents on entry do not matter.
 * Token lists are built on the device (count, scan, stable fill by pair
 * index), so the result is deterministic.  Requires hidden % 256 == 0 and
 * inter % 256 == 0, 1 <= top_k <= n_experts.  The workspace header (its
 * first 256 bytes) holds at QP_MOE_DROPPED_PAIRS_OFFSET the uint32 count of
 * dropped pairs of the call; a call with t == 0 launches nothing and leaves
 * it as it was.
 */
qp_status qp_grouped_expert_gemm(int qtype, const void* w_gate, const void* w_up, const void* w_down,
                                 int64_t n_experts, int64_t hidden, int64_t inter, const uint16_t* x,
                                 int64_t t, int64_t top_k, const int32_t* ids, const float* weights,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Reader of the dropped-pair count of the last qp_grouped_expert_gemm call
 * that used `workspace` (the aprender issue, "Cause": an engine fails closed
 * on input it cannot serve; the count lets the caller do so for expert ids
 * out of range):
 *   workspace (device): that call's workspace, 256-byte aligned.
 *   count (host or device): one uint32_t, written by a copy enqueued on
 *     `stream` after the work already there; valid once the stream has
 *     reached it (pinned host memory or device memory keep the call
 *     asynchronous; for pageable host memory HIP completes the copy first).
 * Errors: QP_ERR_INVALID_PARAMETER for NULL or misaligned pointers,
 * QP_ERR_DEVICE if the copy cannot be enqueued.
 */
#define QP_MOE_DROPPED_PAIRS_OFFSET 0
qp_status qp_grouped_expert_dropped_pairs(const void* workspace, uint32_t* count, hipStream_t stream);

/*
 * Rotary position step on the QK-normed Q or K rows of a chunk, in place
 * (the Strata PR's "Summary": prompt attention over the chunk's Q and K; the
 * pages print no rotary formula, so this is the published rotary embedding in
 * its half-split pairing, the form Qwen3 models use):  for row i (position
 * pos0 + i), head h and j < head_dim / 2, the values a = x[i, h*hd + j] and
 * b = x[i, h*hd + j + hd/2] become
 *   a cos(th) - b sin(th),  a sin(th) + b cos(th),   th = (pos0 + i) * base^(-2j / head_dim)
 * with the angle, cosine, sine and products in binary64 and each result
 * rounded to f32 once.
 *   x (device): t rows of f32, row stride ldx (>= n_head * head_dim), 4-byte
 *               aligned; columns past n_head * head_dim are not touched.
 *   base: the rotary base (1e6 for Qwen3), finite and > 1.
 * Requires head_dim even and <= 1024, n_head <= 4096, 0 <= pos0 <= 2^40.
 * t == 0 is a no-op.  Errors: QP_ERR_INVALID_PARAMETER.
 */
qp_status qp_rope(float* x, int64_t ldx, int64_t t, int64_t n_head, int64_t head_dim, int64_t pos0, double base,
                  hipStream_t stream);

/*
 * Writes the K or V rows of a chunk into a KV cache held as binary16, Q8_0
 * ("INT8") or Q4_0 rows (the Strata PR's "Summary" and the KV table after
 * it): token i, kv head g of src becomes cache row (row0 + i) * n_kv_head + g
 * (row0 = n_past: the cache layout qp_prompt_attention reads).  The pages
 * print no quantizer; each 32 values are stored with the GGUF reference
 * rounding, in binary32:
 *   QP_Q8_0: d = amax / 127, code = x * (1 / d) rounded half away from zero;
 *   QP_Q4_0: d = m / -8 for m the first value of largest magnitude,
 *            code = min(15, trunc(x * (1 / d) + 8.5)) (the product rounded
 *            first), values 16..31 in the high nibbles;
 *   QP_F16W: the nearest-even binary16 of each value;
 * the codes come from the f32 d (0 when d = 0), the block stores the
 * nearest-even binary16 of d.
 *   src (device): t rows of f32 (the k or v projection's output, k after its
 *                 norm and qp_rope), row stride lds (>= n_kv_head * head_dim,
 *                 a multiple of 4), 16-byte aligned.
 *   cache (device): at least (row0 + t) * n_kv_head * qp_row_bytes(kv_type,
 *                 head_dim) bytes, 2-byte aligned (4 for binary16); only the
 *                 chunk's rows are written.
 * Requires head_dim a multiple of 32 and <= 1024, n_kv_head <= 4096, row0 >= 0.
 * t == 0 is a no-op.  Errors: QP_ERR_UNSUPPORTED_TYPE for another kv_type,
 * QP_ERR_INVALID_PARAMETER otherwise.
 */
qp_status qp_kv_cache_write(int kv_type, const float* src, int64_t lds, int64_t t, int64_t n_kv_head,
                            int64_t head_dim, void* cache, int64_t row0, hipStream_t stream);

/*
 * Causal prompt attention of one prefill chunk over a KV cache held as
 * binary16, Q8_0 or Q4_0 rows ("CUDA prefill VRAM loans and SM75 Q4/native-IQ
 * opt-ins", section "Summary" and the KV table after it: prompt attention as
 * a tensor-core path over a quantized KV cache).  The cache holds
 * kv_len = n_past + t tokens (earlier chunks, then this one); query i of the
 * chunk sits at position n_past + i and sees keys 0 .. n_past + i.  Query
 * head h reads kv head h / (n_head / n_kv_head).  For query i, head h:
 *   s_r = scale * (q[i, h] . k[r, g]),  p = softmax_r(s),  out[i, h] = sum_r p_r v[r, g]
 *   kv_type: QP_F16W (binary16 values), QP_Q8_0 (one 34-byte block per 32
 *            values: "INT8" cache rows) or QP_Q4_0 (one 18-byte block per 32
 *            values: binary16 d, then 16 bytes whose low nibbles are values
 *            0..15 and high nibbles values 16..31, each d * (nibble - 8)).
 *            QP_Q4_0 is a KV cache format only: the weight entry points
 *            reject it.
 *   q (device): t rows of f32, row stride ldq floats; head h is columns
 *               h*head_dim .. (h+1)*head_dim-1 (the layout of the q
 *               projection's output).
 *   k_cache, v_cache (device): kv_len * n_kv_head rows of head_dim values in
 *               kv_type, row (r * n_kv_head + g) for token r and kv head g.
 *   out (device): t rows of f32, row stride ldo, head h at h*head_dim.
 * Arithmetic: Q, K, V and the probabilities enter FP16 MFMA products
 * (nearest-even binary16 of the f32 / exact cache values); scores, softmax
 * and accumulation are f32.  scale: a finite number; 0 selects the usual
 * 1 / sqrt(head_dim) (rounded to f32 from the binary64 value).  The running
 * maximum of the online softmax starts at -inf, so any finite scaled scores
 * are handled (scores that overflow f32 give inf or NaN).  Requires
 * head_dim == 128, n_head a multiple of n_kv_head, n_head <= 1024,
 * n_past + t < 2^31, ceil(t/128) * n_head < 2^24 (one workgroup per 128
 * queries and head), ldq and ldo >= n_head*head_dim and multiples of 4, q
 * and out 16-byte aligned, caches 16-byte (F16) or 2-byte (Q8_0, Q4_0)
 * aligned.  t == 0 is a no-op.  out must not overlap q or the caches.  Errors: QP_ERR_UNSUPPORTED_TYPE for another
 * kv_type, QP_ERR_INVALID_PARAMETER otherwise.
 */
qp_status qp_prompt_attention(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                              int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv_head, int64_t head_dim,
                              float scale, float* out, int64_t ldo, hipStream_t stream);

/*
 * Bytes of the workspace qp_prompt_attention_ws takes for a Q8_0 or Q4_0
 * cache of kv_len tokens: the binary16 rows of both caches (0 for any other
 * kv_type or head_dim, kv_len <= 0 or n_kv_head outside 1..1024).  Same
 * passage as qp_prompt_attention.
 */
size_t qp_prompt_attention_workspace_bytes(int kv_type, int64_t kv_len, int64_t n_kv_head, int64_t head_dim);

/*
 * qp_prompt_attention with a workspace (same passage).  For a Q8_0 or Q4_0
 * cache the kv_len * n_kv_head rows of both caches are first decoded into
 * binary16 rows in the workspace (the values the attention itself stages from
 * them, bit for bit: one pass over the caches instead of one per query tile
 * and head), then the attention runs over those rows; the output is bitwise
 * that of qp_prompt_attention.
 *   workspace (device, owned by the caller, 16-byte aligned): at least
 *               qp_prompt_attention_workspace_bytes(kv_type, n_past + t,
 *               n_kv_head, head_dim) bytes; NULL: exactly qp_prompt_attention.
 *               A binary16 cache ignores it.  Calls sharing a workspace must
 *               not run concurrently.
 * Errors: as qp_prompt_attention; QP_ERR_WORKSPACE_TOO_SMALL for a non-NULL
 * workspace below the query, QP_ERR_INVALID_PARAMETER for a misaligned one
 * or a quantized cache of more than 2^27 - 8 rows (kv_len * n_kv_head).
 */
qp_status qp_prompt_attention_ws(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                                 int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv_head, int64_t head_dim,
                                 float scale, float* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Static English name of a status ("QP_OK", ...): the error kinds of the
 * aprender issue's "Cause" (an unsupported type is an InvalidParameter-style
 * error and the call fails closed). */
const char* qp_status_string(qp_status s);

/* Detail of the last error returned on the calling thread (host memory owned
 * by the library, valid until the next call on this thread); same passage. */
const char* qp_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* QPREFILL_H */
