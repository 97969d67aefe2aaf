/*
 * oracle.c -- plain, slow CPU definition of the quantized prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the smoke check and the bench's CPU-baseline
 * leg use it.  It shares no code, header, table or constant generator with the
 * HIP library.
 *
 * What it defines (sources are the three pages, cited by title and section):
 *   - "Qwen3.5 batched prefill has no f32 dequant for IQ2_XXS, IQ3_S, IQ3_XXS,
 *     Q2_K" (aprender issue), section "Cause": every projection weight is
 *     dequantized to f32 before the prefill GEMM, and the f16 mode builds its
 *     f16 copy from that same f32 dequant.  Section "Acceptance (each row)":
 *     the dequant is compared bit for bit with the CPU oracle, including a row
 *     whose last block is partial, and nothing outside the output is written.
 *   - "QK-norm models take the FP16 batched prefill" (aprender PR), section
 *     "What changes": the batched prefill is a chunk of prompt tokens against
 *     each projection, FP16, for models with a per-head QK norm.
 *   - "CUDA prefill VRAM loans and SM75 Q4/native-IQ opt-ins" (Strata PR),
 *     sections "Summary" and "Correctness and safety": the routed experts get
 *     a fused prefill path that chooses and weighs the same experts, and adds
 *     their outputs in the same order, as the unfused path.  Section
 *     "Summary" and the table after it: prompt attention runs over a KV cache
 *     held quantized (Q4_0 or INT8 per row), as a tensor-core path of its own;
 *     the K and V rows of the chunk are written into that cache first, K
 *     after its QK norm and a rotary position step.
 * The pages name the block types but do not print their bit layouts; the
 * layouts below are the GGUF/ggml on-disk convention, restated as formulas.
 *
 * Arithmetic rules: dequant values are computed in binary32, left to right,
 * each operation rounded to nearest-even, with no contraction (build with
 * -ffp-contract=off).  GEMM, QK norm, router and MoE are computed in binary64
 * with sequential sums in the index order of the definition.
 *
 * QP_PLANT=<n> compiles one deliberate mistake (see or_plant_name) so the test
 * suite can show that its pins catch it.  The default build plants nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef QP_PLANT
#define QP_PLANT 0
#endif

#define OR_F16 1
#define OR_Q4_0 2
#define OR_Q8_0 8
#define OR_Q2_K 10
#define OR_Q4_K 12
#define OR_Q5_K 13
#define OR_Q6_K 14

/* Plant codes are macros: #if compares them in the preprocessor. */
#define PLANT_NONE              0
#define PLANT_Q8_UNSIGNED       1  /* Q8_0 quants read as unsigned bytes */
#define PLANT_Q6_NO_OFFSET      2  /* Q6_K quant without the -32 */
#define PLANT_Q6_NO_HIGH        3  /* Q6_K qh bits dropped */
#define PLANT_Q4_SCALE_HIGH     4  /* Q4_K 6-bit scale: high bits of sub-blocks 4..7 dropped */
#define PLANT_SCALE_SELECT      5  /* scale selector off by one sub-block */
#define PLANT_D_FOR_DMIN        6  /* dmin used where d belongs (K types); d ignored (Q8_0, Q6_K) */
#define PLANT_ROW_STRIDE        7  /* floor(cols/QK) blocks per row */
#define PLANT_TAIL              8  /* partial last block written in full */
#define PLANT_F16_RTZ           9  /* f32 -> f16 rounds toward zero */
#define PLANT_F16_SCALE        10  /* d*sc computed in binary16 */
#define PLANT_Q2_NIBBLES       11  /* Q2_K scale/min nibbles swapped */
#define PLANT_Q4_NIBBLE        12  /* Q4_K low/high nibble choice swapped */
#define PLANT_Q6_SHIFT         13  /* Q6_K ql nibble choice taken from the wrong bit of the index */
#define PLANT_GEMM_TRANSPOSE   14  /* Y = X W instead of X W^T */
#define PLANT_GEMM_DROP_K      15  /* last term of each dot product dropped */
#define PLANT_QKN_SUM          16  /* sum of squares instead of mean */
#define PLANT_QKN_EPS          17  /* epsilon dropped */
#define PLANT_QKN_GAIN         18  /* gain indexed by head instead of by column */
#define PLANT_SILU_SIGN        19  /* sigmoid with exp(+g) */
#define PLANT_MOE_WEIGHT       20  /* route weight ignored */
#define PLANT_ROUTER_TIE       21  /* ties go to the higher expert index */
#define PLANT_ROUTER_RENORM    22  /* route weights renormalised over the top-k */
#define PLANT_MOE_UP           23  /* up projection dropped from the product */
#define PLANT_Q5_NO_HIGH       24  /* Q5_K qh bit dropped */
#define PLANT_Q5_HIGH_BIT      25  /* Q5_K qh bit chosen by the nibble half only, not the sub-block */
#define PLANT_F16W_BYTES       26  /* F16 weights read big-endian */
#define PLANT_ATTN_NO_MASK     27  /* queries also attend to later keys */
#define PLANT_ATTN_GQA         28  /* q head h reads kv head h % n_kv instead of h / group */
#define PLANT_ATTN_NO_SCALE    29  /* scores not multiplied by the scale */
#define PLANT_Q4_0_HALVES      30  /* Q4_0: values 0..15 from high nibbles, 16..31 from low */
#define PLANT_Q4_0_OFFSET      31  /* Q4_0 quant without the -8 */
#define PLANT_ATTN_MAX_FLOOR   32  /* softmax maximum taken from a finite floor of -1e30 */
#define PLANT_ROPE_ADJACENT    33  /* RoPE pairs values 2j and 2j+1 instead of j and j + head_dim/2 */
#define PLANT_ROPE_FREQ        34  /* RoPE frequency base^(-j/head_dim) instead of base^(-2j/head_dim) */
#define PLANT_ROPE_SIGN        35  /* RoPE rotates the other way */
#define PLANT_KV_Q8_TRUNC      36  /* Q8_0 cache codes truncated instead of rounded */
#define PLANT_KV_Q4_ABSMAX     37  /* Q4_0 cache scale from |max| / 8 instead of max / -8 */
#define PLANT_KV_Q8_F16_D      38  /* Q8_0 cache codes from the binary16-rounded scale */
#define PLANT_COUNT            39

static const char* const plant_names[PLANT_COUNT] = {
    "none", "q8_unsigned", "q6_no_offset", "q6_no_high", "q4_scale_high",
    "scale_select", "d_for_dmin", "row_stride", "tail", "f16_rtz", "f16_scale",
    "q2_nibbles", "q4_nibble", "q6_shift", "gemm_transpose", "gemm_drop_k",
    "qkn_sum", "qkn_eps", "qkn_gain", "silu_sign", "moe_weight", "router_tie",
    "router_renorm", "moe_up", "q5_no_high", "q5_high_bit", "f16w_bytes",
    "attn_no_mask", "attn_gqa", "attn_no_scale", "q4_0_halves", "q4_0_offset", "attn_max_floor",
    "rope_adjacent", "rope_freq", "rope_sign", "kv_q8_trunc", "kv_q4_absmax", "kv_q8_f16_d"};

int or_plant(void) { return QP_PLANT; }
int or_plant_count(void) { return PLANT_COUNT; }
const char* or_plant_name(int p) { return (p >= 0 && p < PLANT_COUNT) ? plant_names[p] : "?"; }

int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the parallel loops from now on (n >= 1); timing only. */
void or_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary32                                                     */

/* IEEE 754 binary16: sign, 5-bit exponent with bias 15, 10-bit fraction. */
double or_half_to_double(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);              /* zero and subnormals: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + m, e - 25);          /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

float or_half_to_float(uint16_t h) { return (float)or_half_to_double(h); }

/* Round a binary32 value to binary16, nearest with ties to even.
 * |x| is written as q * ulp where ulp is the binary16 spacing at |x|
 * (2^-24 below 2^-14, else 2^(floor(log2|x|) - 10)); q is rounded to an
 * integer n, and n * ulp is encoded.  All steps are exact in binary64. */
uint16_t or_float_to_half(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  double a = fabs((double)f);
  if (isnan(f)) return sign | 0x7E00;
  if (isinf(f)) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e2;                                   /* a = fr * 2^e2, fr in [0.5, 1) */
  frexp(a, &e2);
  int E = e2 - 1;                           /* floor(log2 a) */
  int subnormal = E < -14;
  double ulp = subnormal ? ldexp(1.0, -24) : ldexp(1.0, E - 10);
  double q = a / ulp;                       /* exact: division by a power of two */
  double n = floor(q);
  double frac = q - n;
#if QP_PLANT == PLANT_F16_RTZ
  (void)frac;
#else
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
#endif
  uint32_t bits;
  if (subnormal)
    bits = (uint32_t)n;                     /* n == 1024 encodes 2^-14 exactly */
  else
    bits = ((uint32_t)(E + 15) << 10) + (uint32_t)(n - 1024.0);  /* carry bumps the exponent */
  if (bits >= 0x7C00) bits = 0x7C00;        /* rounds to >= 2^16: overflow to infinity */
  return sign | (uint16_t)bits;
}

void or_half_to_float_array(const uint16_t* src, float* dst, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) dst[i] = or_half_to_float(src[i]);
}

void or_float_to_half_array(const float* src, uint16_t* dst, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) dst[i] = or_float_to_half(src[i]);
}

/* ------------------------------------------------------------------------ */
/* block geometry                                                            */

int64_t or_block_size(int qtype) {
  switch (qtype) {
    case OR_F16: return 1;
    case OR_Q8_0: case OR_Q4_0: return 32;
    case OR_Q4_K: case OR_Q5_K: case OR_Q6_K: case OR_Q2_K: return 256;
    default: return -1;
  }
}

int64_t or_type_size(int qtype) {
  switch (qtype) {
    case OR_F16: return 2;
    case OR_Q8_0: return 34;
    case OR_Q4_0: return 18;
    case OR_Q4_K: return 144;
    case OR_Q5_K: return 176;
    case OR_Q6_K: return 210;
    case OR_Q2_K: return 84;
    default: return -1;
  }
}

static int64_t blocks_per_row(int qtype, int64_t cols) {
  int64_t qk = or_block_size(qtype);
#if QP_PLANT == PLANT_ROW_STRIDE
  return cols / qk;
#else
  return (cols + qk - 1) / qk;
#endif
}

int64_t or_row_bytes(int qtype, int64_t cols) {
  if (or_block_size(qtype) < 0 || cols <= 0) return -1;
  return blocks_per_row(qtype, cols) * or_type_size(qtype);
}

static float f16_at(const uint8_t* p) { return or_half_to_float((uint16_t)(p[0] | (p[1] << 8))); }

/* Round to binary16 and back: only used by the planted binary16-scale fault. */
static float through_f16(float v) { return or_half_to_float(or_float_to_half(v)); }

/* ------------------------------------------------------------------------ */
/* per-type value of weight i (0 <= i < QK) of one block                     */

/* F16 weights (ggml type 1): each "block" is one little-endian binary16
 * value, and the weight is that value (widening to binary32 is exact). */
static float f16w_value(const uint8_t* b) {
#if QP_PLANT == PLANT_F16W_BYTES
  return or_half_to_float((uint16_t)((b[0] << 8) | b[1]));
#else
  return f16_at(b);
#endif
}

/* Q8_0: w = d * q, q the signed byte qs[i]. */
static float q8_0_value(const uint8_t* b, int i) {
  float d = f16_at(b);
#if QP_PLANT == PLANT_Q8_UNSIGNED
  float q = (float)b[2 + i];
#else
  float q = (float)(int8_t)b[2 + i];
#endif
#if QP_PLANT == PLANT_D_FOR_DMIN
  d = 1.0f;
#endif
  return d * q;
}

/* Q4_0 (18 bytes: binary16 d, then 16 bytes of 4-bit quants): value i is
 * d * (q - 8), where q is the low nibble of byte 2 + i for i < 16 and the
 * high nibble of byte 2 + i - 16 for i >= 16.  The pages name Q4_0 as a KV
 * cache format; the layout is the GGUF one. */
static float q4_0_value(const uint8_t* b, int i) {
  float d = f16_at(b);
#if QP_PLANT == PLANT_Q4_0_HALVES
  int q = i < 16 ? (b[2 + i] >> 4) : (b[2 + i - 16] & 0x0F);
#else
  int q = i < 16 ? (b[2 + i] & 0x0F) : (b[2 + i - 16] >> 4);
#endif
#if QP_PLANT == PLANT_Q4_0_OFFSET
  return d * (float)q;
#else
  return d * (float)(q - 8);
#endif
}

/* Q4_K 6-bit (scale, min) of sub-block j from the 12 packed bytes s[0..11]:
 * sub-blocks 0..3 keep their scale in the low 6 bits of s[j] and their min in
 * the low 6 bits of s[j+4]; sub-blocks 4..7 take the low nibble of s[j+4]
 * (scale) or its high nibble (min) as bits 0..3 and the top two bits of s[j-4]
 * (scale) or s[j] (min) as bits 4..5. */
static void q4_k_scale_min(const uint8_t* s, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = s[j] & 63;
    *m = s[j + 4] & 63;
  } else {
#if QP_PLANT == PLANT_Q4_SCALE_HIGH
    *sc = s[j + 4] & 15;
    *m = s[j + 4] >> 4;
#else
    *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
#endif
  }
}

/* Q4_K: sub-block j = i/32 with (sc, m) as above; the quant is a nibble of
 * qs[32*(i/64) + i%32], the low nibble for the first 32 weights of each 64
 * and the high nibble for the next 32.  w = (d*sc)*q - dmin*m. */
static float q4_k_value(const uint8_t* b, int i) {
  float d = f16_at(b), dmin = f16_at(b + 2);
  const uint8_t* scales = b + 4;
  const uint8_t* qs = b + 16;
#if QP_PLANT == PLANT_SCALE_SELECT
  int j = (i / 32 + 1) % 8;
#else
  int j = i / 32;
#endif
  int sc, m;
  q4_k_scale_min(scales, j, &sc, &m);
  uint8_t byte = qs[32 * (i / 64) + i % 32];
#if QP_PLANT == PLANT_Q4_NIBBLE
  int high = (i % 64) < 32;
#else
  int high = (i % 64) >= 32;
#endif
  int q = high ? (byte >> 4) : (byte & 15);
#if QP_PLANT == PLANT_D_FOR_DMIN
  d = dmin;
#endif
  float dsc = d * (float)sc;
#if QP_PLANT == PLANT_F16_SCALE
  dsc = through_f16(dsc);
#endif
  float dm = dmin * (float)m;
  return dsc * (float)q - dm;
}

/* Q5_K: the Q4_K layout with a plane of fifth bits between the scales and
 * the nibbles: d @0, dmin @2, 12 scale bytes @4 (packed as for Q4_K), qh[32]
 * @16, qs[128] @48.  Weight i takes its low four bits from qs exactly as in
 * Q4_K, and its fifth bit from bit i/32 (its sub-block) of qh[i%32].
 * q = low | fifth << 4, in [0, 31].  w = (d*sc)*q - dmin*m. */
static float q5_k_value(const uint8_t* b, int i) {
  float d = f16_at(b), dmin = f16_at(b + 2);
  const uint8_t* scales = b + 4;
  const uint8_t* qh = b + 16;
  const uint8_t* qs = b + 48;
#if QP_PLANT == PLANT_SCALE_SELECT
  int j = (i / 32 + 1) % 8;
#else
  int j = i / 32;
#endif
  int sc, m;
  q4_k_scale_min(scales, j, &sc, &m);
  uint8_t byte = qs[32 * (i / 64) + i % 32];
  int low = (i % 64) >= 32 ? (byte >> 4) : (byte & 15);
#if QP_PLANT == PLANT_Q5_NO_HIGH
  int fifth = 0;
#elif QP_PLANT == PLANT_Q5_HIGH_BIT
  int fifth = (qh[i % 32] >> ((i % 64) / 32)) & 1;
#else
  int fifth = (qh[i % 32] >> (i / 32)) & 1;
#endif
  int q = low | (fifth << 4);
#if QP_PLANT == PLANT_D_FOR_DMIN
  d = dmin;
#endif
  float dsc = d * (float)sc;
#if QP_PLANT == PLANT_F16_SCALE
  dsc = through_f16(dsc);
#endif
  float dm = dmin * (float)m;
  return dsc * (float)q - dm;
}

/* Q6_K: half h = i/128 of the block, r = i%128, quarter c = r/32, l = r%32.
 * Low 4 bits: ql[64h + 32*(c%2) + l], low nibble for c < 2, high for c >= 2.
 * High 2 bits: bits 2c..2c+1 of qh[32h + l].  q = (low | high << 4) - 32.
 * Scale: signed byte scales[i/16].  w = (d*sc)*q. */
static float q6_k_value(const uint8_t* b, int i) {
  const uint8_t* ql = b;
  const uint8_t* qh = b + 128;
  const int8_t* scales = (const int8_t*)(b + 192);
  float d = f16_at(b + 208);
  int h = i / 128, r = i % 128, c = r / 32, l = r % 32;
#if QP_PLANT == PLANT_Q6_SHIFT
  int shift = 4 * (c % 2);
  int low = (ql[64 * h + 32 * (c / 2) + l] >> shift) & 15;
#else
  int low = (ql[64 * h + 32 * (c % 2) + l] >> (4 * (c / 2))) & 15;
#endif
#if QP_PLANT == PLANT_Q6_NO_HIGH
  int high = 0;
#else
  int high = (qh[32 * h + l] >> (2 * c)) & 3;
#endif
#if QP_PLANT == PLANT_Q6_NO_OFFSET
  int q = low | (high << 4);
#else
  int q = (low | (high << 4)) - 32;
#endif
#if QP_PLANT == PLANT_SCALE_SELECT
  int s = (i / 16 + 1) % 16;
#else
  int s = i / 16;
#endif
#if QP_PLANT == PLANT_D_FOR_DMIN
  d = 1.0f;
#endif
  float dsc = d * (float)scales[s];
#if QP_PLANT == PLANT_F16_SCALE
  dsc = through_f16(dsc);
#endif
  return dsc * (float)q;
}

/* Q2_K: half h = i/128, j = (i%128)/32; q = bits 2j..2j+1 of qs[32h + i%32].
 * Scale byte scales[i/16]: low nibble = scale, high nibble = min.
 * w = (d*sc)*q - dmin*m. */
static float q2_k_value(const uint8_t* b, int i) {
  const uint8_t* scales = b;
  const uint8_t* qs = b + 16;
  float d = f16_at(b + 80), dmin = f16_at(b + 82);
  int h = i / 128, j = (i % 128) / 32;
  int q = (qs[32 * h + i % 32] >> (2 * j)) & 3;
#if QP_PLANT == PLANT_SCALE_SELECT
  uint8_t s = scales[(i / 16 + 1) % 16];
#else
  uint8_t s = scales[i / 16];
#endif
#if QP_PLANT == PLANT_Q2_NIBBLES
  int sc = s >> 4, m = s & 15;
#else
  int sc = s & 15, m = s >> 4;
#endif
#if QP_PLANT == PLANT_D_FOR_DMIN
  d = dmin;
#endif
  float dsc = d * (float)sc;
#if QP_PLANT == PLANT_F16_SCALE
  dsc = through_f16(dsc);
#endif
  float dm = dmin * (float)m;
  return dsc * (float)q - dm;
}

static float block_value(int qtype, const uint8_t* b, int i) {
  switch (qtype) {
    case OR_F16: return f16w_value(b);
    case OR_Q8_0: return q8_0_value(b, i);
    case OR_Q4_0: return q4_0_value(b, i);
    case OR_Q4_K: return q4_k_value(b, i);
    case OR_Q5_K: return q5_k_value(b, i);
    case OR_Q6_K: return q6_k_value(b, i);
    default: return q2_k_value(b, i);
  }
}

/* One row of `cols` weights: ceil(cols/QK) whole blocks; the last block's
 * trailing quants beyond `cols` are present in memory and ignored. */
static void dequant_row(int qtype, const uint8_t* row, int64_t cols, float* out) {
  int64_t qk = or_block_size(qtype), ts = or_type_size(qtype);
  int64_t nb = blocks_per_row(qtype, cols);
  for (int64_t blk = 0; blk < nb; ++blk) {
    const uint8_t* b = row + blk * ts;
    for (int64_t i = 0; i < qk; ++i) {
      int64_t c = blk * qk + i;
#if QP_PLANT != PLANT_TAIL
      if (c >= cols) break;
#endif
      out[c] = block_value(qtype, b, (int)i);
    }
  }
}

/* dst[r*cols + c] = value of weight c of row r, for r < rows, c < cols.
 * Returns 0, or -1 for an unsupported type or a bad size. */
int or_dequant_f32(int qtype, const uint8_t* src, int64_t rows, int64_t cols, float* dst) {
  if (or_block_size(qtype) < 0) return -1;
  if (rows < 0 || cols <= 0) return -1;
  int64_t rb = or_row_bytes(qtype, cols);
  /* rows are independent; the PLANT_TAIL build writes past `cols`, so its
   * rows must run in order for the overrun to land deterministically */
#if QP_PLANT == PLANT_TAIL
  for (int64_t r = 0; r < rows; ++r) dequant_row(qtype, src + r * rb, cols, dst + r * cols);
#else
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) dequant_row(qtype, src + r * rb, cols, dst + r * cols);
#endif
  return 0;
}

/* The f16 copy is the binary16 rounding (nearest-even) of the f32 dequant. */
int or_dequant_f16(int qtype, const uint8_t* src, int64_t rows, int64_t cols, uint16_t* dst) {
  if (or_block_size(qtype) < 0) return -1;
  if (rows < 0 || cols <= 0) return -1;
  int64_t rb = or_row_bytes(qtype, cols);
  int64_t qk = or_block_size(qtype);
  int64_t pad = blocks_per_row(qtype, cols) * qk;
#pragma omp parallel
  {
    float* tmp = (float*)malloc(sizeof(float) * (size_t)(pad > cols ? pad : cols));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      dequant_row(qtype, src + r * rb, cols, tmp);
      int64_t n = cols;
#if QP_PLANT == PLANT_TAIL
      if (r == rows - 1) n = pad;
#endif
      for (int64_t c = 0; c < n; ++c) dst[r * cols + c] = or_float_to_half(tmp[c]);
    }
    free(tmp);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* prefill projection: Y[t, n] = sum_k X[t, k] * W[n, k]                     */

static double x_at(const void* x, int x_dtype, int64_t ldx, int64_t t, int64_t k) {
  if (x_dtype == 0) return (double)((const float*)x)[t * ldx + k];
  return or_half_to_double(((const uint16_t*)x)[t * ldx + k]);
}

/* For each token index tok[i] (i < ntok): y[i*n + j] = sum over k (in order
 * 0..K-1, binary64) of X[tok[i], k] * W_f32[j, k], where W_f32 is the exact
 * f32 dequant of W (n rows of K weights).  x_dtype 0 = f32, 1 = binary16.
 * Returns 0, or -1 on a bad argument or allocation failure. */
int or_prefill_gemm(int qtype, const uint8_t* w, int64_t n, int64_t k,
                    const void* x, int x_dtype, int64_t ldx,
                    const int64_t* tok, int64_t ntok, double* y) {
  if (or_block_size(qtype) < 0 || n <= 0 || k <= 0 || ntok < 0 || ldx < k) return -1;
  float* wf = (float*)malloc(sizeof(float) * (size_t)(n * k));
  if (!wf) return -1;
  or_dequant_f32(qtype, w, n, k, wf);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < ntok; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      int64_t t = tok[i];
      double acc = 0.0;
      int64_t kend = k;
#if QP_PLANT == PLANT_GEMM_DROP_K
      kend = k - 1;
#endif
      for (int64_t kk = 0; kk < kend; ++kk) {
#if QP_PLANT == PLANT_GEMM_TRANSPOSE
        double wv = (n == k) ? (double)wf[kk * n + j] : (double)wf[j * k + kk];
#else
        double wv = (double)wf[j * k + kk];
#endif
        acc += x_at(x, x_dtype, ldx, t, kk) * wv;
      }
      y[i * n + j] = acc;
    }
  }
  free(wf);
  return 0;
}

/* Per-head RMSNorm, in place, binary64.  y holds ntok rows of n values; each
 * run of head_dim consecutive columns is one head.  For head h and column j:
 *   y <- y / sqrt(mean_j(y^2) + eps) * gain[h*gain_head_stride + j]
 * gain_head_stride 0 shares one gain vector across heads. */
int or_qknorm(double* y, int64_t ntok, int64_t n, int64_t head_dim,
              const float* gain, int64_t gain_head_stride, double eps) {
  if (head_dim <= 0 || n % head_dim != 0) return -1;
  int64_t heads = n / head_dim;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < ntok; ++i) {
    for (int64_t h = 0; h < heads; ++h) {
      double* v = y + i * n + h * head_dim;
      double ss = 0.0;
      for (int64_t j = 0; j < head_dim; ++j) ss += v[j] * v[j];
#if QP_PLANT == PLANT_QKN_SUM
      double ms = ss;
#else
      double ms = ss / (double)head_dim;
#endif
#if QP_PLANT == PLANT_QKN_EPS
      double r = sqrt(ms);
#else
      double r = sqrt(ms + eps);
#endif
      for (int64_t j = 0; j < head_dim; ++j) {
#if QP_PLANT == PLANT_QKN_GAIN
        double g = (double)gain[h * gain_head_stride + (h % head_dim)];
#else
        double g = (double)gain[h * gain_head_stride + j];
#endif
        v[j] = v[j] / r * g;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* routed experts                                                            */

/* Router, binary64: p = softmax(logits[t, :]) over the experts; the top_k
 * experts by logit, largest first, ties to the lower expert index;
 * weight = p of the chosen expert (renorm != 0 divides by the sum of the
 * chosen p).  ids and weights are [t][top_k]. */
int or_route_topk(const float* logits, int64_t t, int64_t e, int64_t top_k, int renorm,
                  int32_t* ids, double* weights) {
  if (t < 0 || e <= 0 || top_k <= 0 || top_k > e) return -1;
#if QP_PLANT == PLANT_ROUTER_RENORM
  renorm = 1;
#endif
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)e);
    char* taken = (char*)malloc((size_t)e);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < t; ++i) {
      const float* l = logits + i * e;
      double mx = -INFINITY;
      for (int64_t j = 0; j < e; ++j) if ((double)l[j] > mx) mx = (double)l[j];
      double sum = 0.0;
      for (int64_t j = 0; j < e; ++j) { p[j] = exp((double)l[j] - mx); sum += p[j]; }
      for (int64_t j = 0; j < e; ++j) p[j] /= sum;
      memset(taken, 0, (size_t)e);
      double chosen = 0.0;
      for (int64_t s = 0; s < top_k; ++s) {
        int64_t best = -1;
        for (int64_t j = 0; j < e; ++j) {
          if (taken[j]) continue;
#if QP_PLANT == PLANT_ROUTER_TIE
          if (best < 0 || l[j] >= l[best]) best = j;
#else
          if (best < 0 || l[j] > l[best]) best = j;
#endif
        }
        taken[best] = 1;
        ids[i * top_k + s] = (int32_t)best;
        weights[i * top_k + s] = p[best];
        chosen += p[best];
      }
      if (renorm)
        for (int64_t s = 0; s < top_k; ++s) weights[i * top_k + s] /= chosen;
    }
    free(p);
    free(taken);
  }
  return 0;
}

/* Routed expert FFN for the tokens tok[0..ntok), binary64:
 *   for slot s of token t with expert e = ids[t][s]:
 *     g = X[t] . Wg_e^T,  u = X[t] . Wu_e^T          (inter values each)
 *     h = g / (1 + exp(-g)) * u                       (SiLU(g) * u)
 *     d = h . Wd_e^T                                  (hidden values)
 *   out[i] = sum over s = 0..top_k-1, in slot order, of weights[t][s] * d_s
 * Expert e's gate/up tensors are inter rows of hidden weights starting at
 * e * inter * row_bytes(hidden); its down tensor is hidden rows of inter
 * weights starting at e * hidden * row_bytes(inter).  X is binary16. */
int or_moe(int qtype, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
           int64_t n_experts, int64_t hidden, int64_t inter,
           const uint16_t* x, int64_t ldx, int64_t top_k,
           const int32_t* ids, const double* weights,
           const int64_t* tok, int64_t ntok, double* out) {
  if (or_block_size(qtype) < 0 || n_experts <= 0 || hidden <= 0 || inter <= 0 || top_k <= 0)
    return -1;
  int64_t rb_h = or_row_bytes(qtype, hidden), rb_i = or_row_bytes(qtype, inter);
  int64_t gate_stride = inter * rb_h, down_stride = hidden * rb_i;
  for (int64_t i = 0; i < ntok; ++i)
    for (int64_t s = 0; s < top_k; ++s) {
      int32_t e = ids[tok[i] * top_k + s];
      if (e < 0 || e >= n_experts) return -1;
    }
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)(hidden > inter ? hidden : inter));
    double* xd = (double*)malloc(sizeof(double) * (size_t)hidden);
    double* h = (double*)malloc(sizeof(double) * (size_t)inter);
#pragma omp for schedule(dynamic)
    for (int64_t i = 0; i < ntok; ++i) {
      int64_t t = tok[i];
      double* o = out + i * hidden;
      for (int64_t c = 0; c < hidden; ++c) xd[c] = or_half_to_double(x[t * ldx + c]);
      for (int64_t c = 0; c < hidden; ++c) o[c] = 0.0;
      for (int64_t s = 0; s < top_k; ++s) {
        int32_t e = ids[t * top_k + s];
        double wgt = weights[t * top_k + s];
#if QP_PLANT == PLANT_MOE_WEIGHT
        wgt = 1.0;
#endif
        for (int64_t j = 0; j < inter; ++j) {
          double g = 0.0, u = 0.0;
          dequant_row(qtype, wg + e * gate_stride + j * rb_h, hidden, wrow);
          for (int64_t c = 0; c < hidden; ++c) g += xd[c] * (double)wrow[c];
          dequant_row(qtype, wu + e * gate_stride + j * rb_h, hidden, wrow);
          for (int64_t c = 0; c < hidden; ++c) u += xd[c] * (double)wrow[c];
#if QP_PLANT == PLANT_SILU_SIGN
          double silu = g / (1.0 + exp(g));
#else
          double silu = g / (1.0 + exp(-g));
#endif
#if QP_PLANT == PLANT_MOE_UP
          h[j] = silu;
#else
          h[j] = silu * u;
#endif
        }
        for (int64_t c = 0; c < hidden; ++c) {
          dequant_row(qtype, wd + e * down_stride + c * rb_i, inter, wrow);
          double dv = 0.0;
          for (int64_t j = 0; j < inter; ++j) dv += h[j] * (double)wrow[j];
          o[c] += wgt * dv;
        }
      }
    }
    free(wrow);
    free(xd);
    free(h);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* prompt attention                                                          */

/* Causal prompt attention of one chunk over a quantized KV cache, binary64
 * ("CUDA prefill VRAM loans and SM75 Q4/native-IQ opt-ins", section
 * "Summary" and the KV table after it: prompt attention over a KV cache
 * stored as quantized rows).  The cache holds kv_len = n_past + t tokens;
 * the row of token r and kv head g starts at byte (r*n_kv + g)*row_bytes(
 * kvtype, head_dim) of kc (keys) and vc (values) and decodes as a weight row
 * does.  Query i of the chunk (i < t) sits at position n_past + i and sees
 * keys 0 .. n_past + i.  Query head h reads kv head h / (n_head / n_kv)
 * (grouped-query attention).  For each sampled query i = tok[..] and head h:
 *   s_r = scale * (q[i, h] . k[r, g])            r = 0 .. n_past + i
 *   p_r = exp(s_r - max_r s_r) / sum_r exp(s_r - max_r s_r)
 *   out[i, h] = sum_r p_r v[r, g]
 * q is f32 with row stride ldq; head h is columns h*head_dim ..
 * out is [ntok][n_head*head_dim]. */
int or_attention(int kvtype, const float* q, int64_t ldq, const uint8_t* kc, const uint8_t* vc,
                 int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv, int64_t head_dim,
                 double scale, const int64_t* tok, int64_t ntok, double* out) {
  if (or_block_size(kvtype) < 0 || n_past < 0 || t < 0 || n_head <= 0 || n_kv <= 0 ||
      n_head % n_kv != 0 || head_dim <= 0 || head_dim % or_block_size(kvtype) != 0)
    return -1;
  for (int64_t i = 0; i < ntok; ++i)
    if (tok[i] < 0 || tok[i] >= t) return -1;
  const int64_t kv_len = n_past + t, group = n_head / n_kv;
  const int64_t rb = or_row_bytes(kvtype, head_dim);
#if QP_PLANT == PLANT_ATTN_NO_SCALE
  scale = 1.0;
#endif
  /* decode the whole cache once (values in binary32, exact, as for weights) */
  float* kf = (float*)malloc(sizeof(float) * (size_t)(kv_len * n_kv * head_dim + 1));
  float* vf = (float*)malloc(sizeof(float) * (size_t)(kv_len * n_kv * head_dim + 1));
  for (int64_t r = 0; r < kv_len * n_kv; ++r) {
    dequant_row(kvtype, kc + r * rb, head_dim, kf + r * head_dim);
    dequant_row(kvtype, vc + r * rb, head_dim, vf + r * head_dim);
  }
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)kv_len);
#pragma omp for collapse(2) schedule(dynamic)
    for (int64_t i = 0; i < ntok; ++i) {
      for (int64_t h = 0; h < n_head; ++h) {
#if QP_PLANT == PLANT_ATTN_GQA
        const int64_t g = h % n_kv;
#else
        const int64_t g = h / group;
#endif
#if QP_PLANT == PLANT_ATTN_NO_MASK
        const int64_t last = kv_len - 1;
#else
        const int64_t last = n_past + tok[i];
#endif
        const float* qi = q + tok[i] * ldq + h * head_dim;
#if QP_PLANT == PLANT_ATTN_MAX_FLOOR
        double mx = -1e30;
#else
        double mx = -INFINITY;
#endif
        for (int64_t r = 0; r <= last; ++r) {
          const float* kr = kf + (r * n_kv + g) * head_dim;
          double dot = 0.0;
          for (int64_t j = 0; j < head_dim; ++j) dot += (double)qi[j] * (double)kr[j];
          s[r] = scale * dot;
          if (s[r] > mx) mx = s[r];
        }
        double sum = 0.0;
        for (int64_t r = 0; r <= last; ++r) { s[r] = exp(s[r] - mx); sum += s[r]; }
        double* o = out + (i * n_head + h) * head_dim;
        for (int64_t j = 0; j < head_dim; ++j) o[j] = 0.0;
        for (int64_t r = 0; r <= last; ++r) {
          const float* vr = vf + (r * n_kv + g) * head_dim;
          const double p = s[r] / sum;
          for (int64_t j = 0; j < head_dim; ++j) o[j] += p * (double)vr[j];
        }
      }
    }
    free(s);
  }
  free(kf);
  free(vf);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Rotary position step and KV cache rows                                     */

/* Rotary position embedding, in place, of t rows of n_head heads of head_dim
 * f32 values (row stride ldx), row i at position pos0 + i.  Reading: the
 * pages name a rotary step after the QK norm but print no formula; this is
 * the rotation of the published rotary embedding in its half-split pairing
 * (the one Qwen3 models use): for j < head_dim / 2, values j and
 * j + head_dim / 2 of a head form a pair turned by the angle
 * (pos0 + i) * base^(-2j / head_dim).  Angle, cosine, sine and the two
 * products are binary64; each result is rounded to f32 once. */
int or_rope(float* x, int64_t ldx, int64_t t, int64_t n_head, int64_t head_dim, int64_t pos0, double base) {
  if (t < 0 || n_head <= 0 || head_dim <= 0 || head_dim % 2 != 0 || ldx < n_head * head_dim || pos0 < 0 ||
      !(base > 0.0))
    return -1;
  const int64_t half = head_dim / 2;
  for (int64_t i = 0; i < t; ++i) {
    const double pos = (double)(pos0 + i);
    for (int64_t h = 0; h < n_head; ++h) {
      float* v = x + i * ldx + h * head_dim;
      for (int64_t j = 0; j < half; ++j) {
#if QP_PLANT == PLANT_ROPE_FREQ
        const double theta = pos * pow(base, -(double)j / (double)head_dim);
#else
        const double theta = pos * pow(base, -2.0 * (double)j / (double)head_dim);
#endif
        const double c = cos(theta), sn = sin(theta);
#if QP_PLANT == PLANT_ROPE_ADJACENT
        const int64_t ia = 2 * j, ib = 2 * j + 1;
#else
        const int64_t ia = j, ib = j + half;
#endif
        const double a = (double)v[ia], b = (double)v[ib];
#if QP_PLANT == PLANT_ROPE_SIGN
        v[ia] = (float)(a * c + b * sn);
        v[ib] = (float)(b * c - a * sn);
#else
        v[ia] = (float)(a * c - b * sn);
        v[ib] = (float)(a * sn + b * c);
#endif
      }
    }
  }
  return 0;
}

static void put_half(uint8_t* p, uint16_t h) {
  p[0] = (uint8_t)(h & 0xFF);
  p[1] = (uint8_t)(h >> 8);
}

/* Q8_0 block of 32 f32 values.  Reading (the pages name an INT8 cache but
 * print no quantizer): the GGUF reference rounding, in binary32: the scale
 * d = amax / 127 for amax the largest |x|, each code the nearest integer of
 * x * (1/d), halves away from zero (0 when d = 0); the block stores the
 * nearest-even binary16 of d, while the codes come from the f32 d. */
static void q8_0_block(const float* x, uint8_t* b) {
  float amax = 0.0f;
  for (int j = 0; j < 32; ++j) {
    const float a = fabsf(x[j]);
    if (a > amax) amax = a;
  }
  const float d = amax / 127.0f;
#if QP_PLANT == PLANT_KV_Q8_F16_D
  const float dq = or_half_to_float(or_float_to_half(d));
  const float id = dq != 0.0f ? 1.0f / dq : 0.0f;
#else
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
#endif
  put_half(b, or_float_to_half(d));
  for (int j = 0; j < 32; ++j) {
    const float v = x[j] * id;
#if QP_PLANT == PLANT_KV_Q8_TRUNC
    b[2 + j] = (uint8_t)(int8_t)(int)v;
#else
    b[2 + j] = (uint8_t)(int8_t)(int)roundf(v);
#endif
  }
}

/* Q4_0 block of 32 f32 values.  Reading, as for Q8_0, the GGUF reference
 * rounding in binary32: m is the first value of largest magnitude, d = m / -8,
 * each code the integer part of x * (1/d) + 8.5 (the product rounded before
 * the sum), at most 15 (0 when d = 0 gives code 8); codes of values 0..15 go
 * to the low nibbles of bytes 2..17, values 16..31 to the high nibbles. */
static void q4_0_block(const float* x, uint8_t* b) {
  float amax = 0.0f, m = 0.0f;
  for (int j = 0; j < 32; ++j) {
    if (fabsf(x[j]) > amax) {
      amax = fabsf(x[j]);
      m = x[j];
    }
  }
#if QP_PLANT == PLANT_KV_Q4_ABSMAX
  const float d = amax / 8.0f;
#else
  const float d = m / -8.0f;
#endif
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
  put_half(b, or_float_to_half(d));
  int q[32];
  for (int j = 0; j < 32; ++j) {
    const float p = x[j] * id;
    const float v = p + 8.5f;
    int c = (int)v;
    q[j] = c > 15 ? 15 : c;
  }
  for (int j = 0; j < 16; ++j) b[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
}

/* The cache rows of t tokens: token i, kv head g of src (row stride lds,
 * head g at column g * head_dim) becomes cache row i * n_kv + g, in kvtype
 * (F16: the nearest-even binary16 of each value; Q8_0 and Q4_0 as above),
 * rows back to back in dst. */
int or_kv_quantize(int kvtype, const float* src, int64_t lds, int64_t t, int64_t n_kv, int64_t head_dim,
                   uint8_t* dst) {
  if ((kvtype != OR_F16 && kvtype != OR_Q8_0 && kvtype != OR_Q4_0) || t < 0 || n_kv <= 0 || head_dim <= 0 ||
      head_dim % 32 != 0 || lds < n_kv * head_dim)
    return -1;
  const int64_t rb = or_row_bytes(kvtype, head_dim);
  for (int64_t i = 0; i < t; ++i)
    for (int64_t g = 0; g < n_kv; ++g) {
      const float* x = src + i * lds + g * head_dim;
      uint8_t* row = dst + (i * n_kv + g) * rb;
      for (int64_t c = 0; c < head_dim; c += 32) {
        if (kvtype == OR_F16) {
          for (int j = 0; j < 32; ++j) put_half(row + 2 * (c + j), or_float_to_half(x[c + j]));
        } else if (kvtype == OR_Q8_0) {
          q8_0_block(x + c, row + (c / 32) * 34);
        } else {
          q4_0_block(x + c, row + (c / 32) * 18);
        }
      }
    }
  return 0;
}
