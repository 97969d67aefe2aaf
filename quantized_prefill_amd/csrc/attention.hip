// attention.hip -- causal prompt attention of one prefill chunk over a KV
// cache held as binary16, Q8_0 or Q4_0 rows ("CUDA prefill VRAM loans and SM75
// Q4/native-IQ opt-ins", section "Summary" and the KV table after it: prompt
// attention as a tensor-core path over a quantized KV cache).
//
// One workgroup = 128 queries of one query head: 4 waves of 32 queries
// (NH = 1), or two halves of 4 such waves with the same queries (NH = 2).
// The keys of the head's kv head stream through LDS in blocks of 64: half h
// takes blocks h, h + NH, h + 2 NH, .. into its own double buffer, K as rows
// (64 x 128), V transposed (128 x 64), both binary16, decoded from the cache
// as they are staged.  With two halves, the second hands its running
// maximum, row-sum share and O through LDS to the first at the end, which
// merges the two (the usual rescale of both by 2^(m_h - max)) and stores.
// Two halves keep a CU at two waves per SIMD for the whole of every tile,
// whatever the tiles' lengths: the choice for a launch of one round, where
// the causal tiles' lengths differ up to the grid size and nothing else
// evens them out; with several rounds, single halves (two workgroups per
// CU, no shared barrier) are faster.  Per wave and key block:
//   S^T (64 keys x 32 queries) = K . Q^T    16 v_mfma_f32_32x32x16_f16
//   online softmax over the keys            one lane owns one query column
//   O^T (128 x 32) += V^T . P^T             16 v_mfma_f32_32x32x16_f16
// Forming S transposed puts each query's scores in one lane (16 per 32-key
// tile, plus the partner lane 32 apart), so the row maximum costs a single
// cross-lane step, the rescale of O^T is a per-lane multiply, and the
// probabilities feed the second product as its B operand straight from the
// accumulator registers (the key order inside a 16-key step is the
// accumulator's row order; V^T is read in that order).
//
// Numerics: Q is rounded to binary16 (nearest even; negated for a negative
// scale), K and V are the exact cache values rounded to binary16, scores and
// the softmax are f32 (exp2 of scale*log2(e)-scaled scores, the scaling and
// the running maximum's subtraction one fma while the maxima are within
// 1024), P is rounded to binary16 for the second product, O accumulates in
// f32 and is divided by the f32 row sum.
#include "qp_device.h"
#include "qp_internal.h"

namespace qp {
namespace {

constexpr int kD = 128;              // head dim
constexpr int kWaves = 4;            // per half
constexpr int kBM = 32 * kWaves;     // queries per workgroup
constexpr int kBK = 64;              // keys per staged block
constexpr int kKP = kD + 8;          // K row pitch in halves: 16-lane reads hit distinct banks
constexpr int kVP = kD + 32;         // V row pitch in halves: 80 dwords, so the 4 key rows of a 32-lane
                                     // transposed read fall in 4 disjoint 16-bank groups
constexpr int kStage = kBK * kKP + kBK * kVP;  // halves per stage

struct AttnArgs {
  const float* q;
  const uint8_t* kc;
  const uint8_t* vc;
  float* o;
  int64_t ldq, ldo;
  int n_past, t, kv_len;
  int n_head, n_kv, group;
  int nqt;     // query tiles of 128
  int xcd;     // 1: the workgroups of one kv group go to one XCD
  float c;     // scale * log2(e)
};

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// 8 consecutive cache values of one row (a chunk), raw, then as binary16.
template <int KV> struct Chunk;

template <> struct Chunk<kF16> {
  static constexpr int64_t kRowBytes = 2 * kD;
  u32x4 raw;
  __device__ __forceinline__ void load(const uint8_t* row, int dc) { raw = *(const u32x4*)(row + 16 * dc); }
  __device__ __forceinline__ void zero() { raw = (u32x4){0, 0, 0, 0}; }
  __device__ __forceinline__ u32x4 halves() const { return raw; }
};

template <> struct Chunk<kQ8_0> {
  static constexpr int64_t kRowBytes = 34 * (kD / 32);
  uint32_t d, q0, q1;
  __device__ __forceinline__ void load(const uint8_t* row, int dc) {
    const uint16_t* b = (const uint16_t*)(row + 34 * (dc >> 2));  // rows and blocks start on even bytes
    const uint16_t* qs = b + 1 + 4 * (dc & 3);
    d = b[0];
    q0 = (uint32_t)qs[0] | ((uint32_t)qs[1] << 16);
    q1 = (uint32_t)qs[2] | ((uint32_t)qs[3] << 16);
  }
  __device__ __forceinline__ void zero() { d = q0 = q1 = 0; }
  __device__ __forceinline__ u32x4 halves() const {
    const float s = f16_to_f32(d);
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = s * (float)(int8_t)(q0 >> (8 * e));
      v[4 + e] = s * (float)(int8_t)(q1 >> (8 * e));
    }
    return (u32x4){pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])};
  }
};

// Q4_0: 18-byte blocks (binary16 d, 16 bytes of nibbles); value j of a block
// is d * (q - 8) with q the low nibble of byte j (j < 16) or the high nibble
// of byte j - 16.  Chunk dc holds values 8 (dc & 3) .. of block dc >> 2: the
// low nibbles of bytes 8 (dc & 1) .. for dc & 3 < 2, else their high nibbles.
template <> struct Chunk<kQ4_0> {
  static constexpr int64_t kRowBytes = 18 * (kD / 32);
  uint32_t d, q0, q1, hi;
  __device__ __forceinline__ void load(const uint8_t* row, int dc) {
    const uint16_t* b = (const uint16_t*)(row + 18 * (dc >> 2));  // rows and blocks start on even bytes
    const uint16_t* qs = b + 1 + 4 * (dc & 1);
    d = b[0];
    q0 = (uint32_t)qs[0] | ((uint32_t)qs[1] << 16);
    q1 = (uint32_t)qs[2] | ((uint32_t)qs[3] << 16);
    hi = (dc & 2) ? 4u : 0u;
  }
  __device__ __forceinline__ void zero() { d = q0 = q1 = hi = 0; }
  __device__ __forceinline__ u32x4 halves() const {
    const float s = f16_to_f32(d);
    const uint32_t n0 = (q0 >> hi) & 0x0F0F0F0Fu, n1 = (q1 >> hi) & 0x0F0F0F0Fu;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = s * (float)((int)((n0 >> (8 * e)) & 0xFu) - 8);
      v[4 + e] = s * (float)((int)((n1 >> (8 * e)) & 0xFu) - 8);
    }
    return (u32x4){pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])};
  }
};

template <int KV, int NH>
__global__ __launch_bounds__(64 * kWaves * NH) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(AttnArgs p) {
  using C = Chunk<KV>;
  __shared__ __attribute__((aligned(16))) _Float16 smem[NH * 2 * kStage];
  const int half = NH == 1 ? 0 : (int)(threadIdx.x >> 8);  // wave-uniform
  const int tid = threadIdx.x & 255;          // thread within the half
  const int lane = tid & 63, wave = tid >> 6;  // wave within the half
  const int r = lane & 31, hh = lane >> 5;
  _Float16* const lds = smem + half * 2 * kStage;  // the half's double buffer

  // workgroup -> (query tile, head); the longest tiles first.  With the XCD
  // map, the group's query heads of one (tile, kv head) unit are dispatched
  // back to back on one XCD (block b runs on XCD b % 8) and share its L2.
  int unit, member;
  const int b = blockIdx.x;
  if (p.xcd) {
    const int slot = b >> 3;
    member = slot % p.group;
    unit = (slot / p.group) * 8 + (b & 7);
  } else {
    unit = b / p.group;
    member = b % p.group;
  }
  const int qt = p.nqt - 1 - unit / p.n_kv;
  const int g = unit % p.n_kv;
  const int head = g * p.group + member;
  const int q0 = qt * kBM;
  const int q0w = q0 + 32 * wave;
  const bool wave_live = q0w < p.t;

  // this wave's queries as the B operand of K . Q^T: query r, dims 16c + 8hh ..
  // A negative scale negates Q (exact) so that the scores are scaled by
  // csc = |scale| log2(e) > 0 (or 0) in the log2 domain.
  const float csc = __builtin_fabsf(p.c);
  const float qsign = p.c < 0.f ? -1.f : 1.f;
  half8 qf[8];
  {
    const int qi = q0w + r;
    const float* qrow = p.q + (int64_t)qi * p.ldq + (int64_t)head * kD + 8 * hh;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float4v a = {0, 0, 0, 0}, bq = {0, 0, 0, 0};
      if (qi < p.t) {
        a = *(const float4v*)(qrow + 16 * c) * qsign;
        bq = *(const float4v*)(qrow + 16 * c + 4) * qsign;
      }
      const u32x4 h = {pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]), pack_f16x2(bq[0], bq[1]),
                       pack_f16x2(bq[2], bq[3])};
      qf[c] = __builtin_bit_cast(half8, h);
    }
  }

  const int last_q = (q0 + kBM - 1 < p.t - 1) ? q0 + kBM - 1 : p.t - 1;
  const int nkb = (p.n_past + last_q) / kBK + 1;
  const int64_t row_stride = (int64_t)p.n_kv * C::kRowBytes;
  const uint8_t* kbase = p.kc + (int64_t)g * C::kRowBytes;
  const uint8_t* vbase = p.vc + (int64_t)g * C::kRowBytes;

  // staging.  K and V chunk j of this thread: key (tid + 256 j) >> 4, dims
  // 8 * (tid & 15) ..  (16 lanes read one row); both stored as rows, V^T's
  // operands come from V's rows by transposed reads.
  C kch[4], vch[4];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kb * kBK + ((tid + 256 * j) >> 4);
      if (key < p.kv_len)
        kch[j].load(kbase + key * row_stride, tid & 15);
      else
        kch[j].zero();
      if (key < p.kv_len)
        vch[j].load(vbase + key * row_stride, tid & 15);
      else
        vch[j].zero();
    }
  };
  auto store_block = [&](int buf) {
    _Float16* ks = lds + buf * kStage;
    _Float16* vs = ks + kBK * kKP;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (tid + 256 * j) >> 4;
      *(u32x4*)(ks + row * kKP + 8 * (tid & 15)) = kch[j].halves();
      *(u32x4*)(vs + row * kVP + 8 * (tid & 15)) = vch[j].halves();
    }
  };

  float16v o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 16; ++a) o[dt][a] = 0.0f;
  // -inf until the first block: every live query sees key 0 there, so the
  // running maximum is finite from then on, whatever the (finite) scores
  float m_run = -INFINITY;
  float l_part = 0.0f;   // this lane's share of the row sum (its 16 key rows per tile)
  const int qpos_lo = p.n_past + q0w;
  const int qpos = qpos_lo + r;

  // half h: blocks h + NH i, i < niter (the second half may have one fewer)
  const int niter = (nkb + NH - 1) / NH;
  if (half < nkb) {
    load_block(half);
    store_block(0);
  }
  __syncthreads();
  for (int i = 0; i < niter; ++i) {
    const int kb = NH * i + half;
    if (kb + NH < nkb) load_block(kb + NH);
    const int key0 = kb * kBK;
    if (kb < nkb && wave_live && key0 <= qpos_lo + 31) {
      const _Float16* ks = lds + (i & 1) * kStage;
      const _Float16* vs = ks + kBK * kKP;
      float16v s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int a = 0; a < 16; ++a) s[kt][a] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const half8 ka = *(const half8*)(ks + (32 * kt + r) * kKP + 16 * c + 8 * hh);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[c], s[kt], 0, 0, 0);
        }
      }
      // keys after the query to -inf (only blocks on the diagonal have any;
      // the test is wave-uniform), then the block maximum of the raw scores:
      // with csc > 0 the scaled maximum is csc times it, the same f32 value
      // as the largest of the rounded products
      if (key0 + kBK - 1 > qpos_lo) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int a = 0; a < 16; ++a)
            if (key0 + 32 * kt + 8 * (a >> 2) + 4 * hh + (a & 3) > qpos) s[kt][a] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s[kt][a]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_blk = mx == -INFINITY ? -INFINITY : mx * csc;
      // The running maximum moves only in a block where some query of the
      // wave sees a scaled score more than 8 above it (always at its first
      // visible key): in the others p is at most 2^8, which binary16 holds at
      // full precision, and O and the row sums need no rescale.
      if (__any(m_blk > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, m_blk);
        // a row with no visible key yet keeps -inf and subtracts 0 instead,
        // so that exp2 sees -inf, never -inf - -inf
        const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int a = 0; a < 16; ++a) o[dt][a] *= alpha;
        m_run = m_new;
      }
      const float m_sub = m_run == -INFINITY ? 0.f : m_run;
      // p = 2^(csc s - m).  With |m| <= 1024 for every query of the wave, one
      // fma: it differs from the rounded product minus m by at most half an
      // ulp of m (2^-14), far below P's binary16 rounding.  Otherwise the
      // rounded product first, so that the maximum's own p is exactly 1
      // however large the scores.
      const bool fused = __all(__builtin_fabsf(m_sub) <= 1024.f);
      float pv[32];
      if (fused) {
#pragma unroll
        for (int e = 0; e < 32; ++e) pv[e] = __builtin_fmaf(s[e >> 4][e & 15], csc, -m_sub);
      } else {
#pragma clang fp contract(off)
#pragma unroll
        for (int e = 0; e < 32; ++e) pv[e] = s[e >> 4][e & 15] * csc - m_sub;
      }
      half8 pb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[8 * st + e] = __builtin_amdgcn_exp2f(pv[8 * st + e]);
          l_part += pv[8 * st + e];
        }
        const float* q8 = pv + 8 * st;
        const u32x4 h = {pack_f16x2(q8[0], q8[1]), pack_f16x2(q8[2], q8[3]), pack_f16x2(q8[4], q8[5]),
                         pack_f16x2(q8[6], q8[7])};
        pb[st] = __builtin_bit_cast(half8, h);
      }
      // k index 8hh + e of step st is key 16 st + 8 (e >> 2) + 4 hh + (e & 3).
      // The A operand (dim l % 32, those 8 keys) by two transposed reads of V
      // rows: in each 16-lane group, lane m addresses row K0 + m / 4, dims
      // D + 4 (m % 4) .. + 3, and lane j receives rows K0 .. K0 + 3 of dim
      // D + j (D = 32 dt + 16 ((l >> 4) & 1), K0 = 16 st + 4 hh and + 8).
      const _Float16* vl = vs + (4 * hh + ((lane & 15) >> 2)) * kVP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          typedef short s4 __attribute__((ext_vector_type(4)));
          const _Float16* vr = vl + 16 * st * kVP + 32 * dt;
          const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)vr);
          const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vr + 8 * kVP));
          const half4 l4 = __builtin_bit_cast(half4, lo), h4 = __builtin_bit_cast(half4, hi);
          const half8 va = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[st], o[dt], 0, 0, 0);
        }
    }
    if (kb + NH < nkb) store_block((i + 1) & 1);
    __syncthreads();
  }

  // merge: the second half's m, row-sum share and O go through LDS (66 floats
  // per lane, lane-minor, so that every access is one dword per lane)
  float* xch = (float*)smem + wave * 66 * 64 + lane;
  if (NH == 2 && half == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 16; ++a) xch[(16 * dt + a) * 64] = o[dt][a];
    xch[64 * 64] = m_run;
    xch[65 * 64] = l_part;
  }
  if (NH == 2) __syncthreads();
  if (half == 1) return;
  if (NH == 2) {
    const float m_b = xch[64 * 64], l_b = xch[65 * 64];
    const float m = fmaxf(m_run, m_b);  // finite for a live query: key 0 is in the first half's block 0
    const float m_s = m == -INFINITY ? 0.f : m;
    const float fa = __builtin_amdgcn_exp2f(m_run - m_s), fb = __builtin_amdgcn_exp2f(m_b - m_s);
    l_part = l_part * fa + l_b * fb;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 16; ++a) o[dt][a] = o[dt][a] * fa + xch[(16 * dt + a) * 64] * fb;
  }

  const float l = l_part + __shfl_xor(l_part, 32, 64);
  const int qi = q0w + r;
  if (!wave_live || qi >= p.t) return;
  const float inv = 1.0f / l;
  float* orow = p.o + (int64_t)qi * p.ldo + (int64_t)head * kD + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4v*)(orow + 32 * dt + 8 * i) = (float4v){o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv,
                                                       o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv};
}

// Two quantized caches' rows (K, then V) as binary16 rows (the values the
// attention kernel's own staging makes of them, bit for bit): one thread
// per 8 values, rows of kD values.
template <int KV>
__global__ __launch_bounds__(256) void kv_decode_f16_kernel(const uint8_t* __restrict__ src0,
                                                            const uint8_t* __restrict__ src1, int64_t rows,
                                                            u32x4* __restrict__ dst0, u32x4* __restrict__ dst1) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk of 8 values
  const int64_t per = rows * (kD / 8);
  const bool second = i >= per;
  if (second) i -= per;
  if (i >= per) return;
  const int64_t row = i / (kD / 8);
  const int dc = (int)(i - row * (kD / 8));
  Chunk<KV> c;
  c.load((second ? src1 : src0) + row * Chunk<KV>::kRowBytes, dc);
  (second ? dst1 : dst0)[i] = c.halves();
}

}  // namespace

int64_t attention_row_bytes(int kv_type) {
  switch (kv_type) {
    case kF16: return Chunk<kF16>::kRowBytes;
    case kQ8_0: return Chunk<kQ8_0>::kRowBytes;
    case kQ4_0: return Chunk<kQ4_0>::kRowBytes;
    default: return -1;
  }
}

hipError_t launch_kv_decode_f16(int kv_type, const void* k_src, const void* v_src, int64_t rows, void* k_dst,
                                void* v_dst, hipStream_t s) {
  const int64_t chunks = 2 * rows * (kD / 8);
  if (chunks == 0) return hipSuccess;
  const dim3 grid((uint32_t)((chunks + 255) / 256));
  if (kv_type == kQ8_0)
    hipLaunchKernelGGL(kv_decode_f16_kernel<kQ8_0>, grid, dim3(256), 0, s, (const uint8_t*)k_src,
                       (const uint8_t*)v_src, rows, (u32x4*)k_dst, (u32x4*)v_dst);
  else if (kv_type == kQ4_0)
    hipLaunchKernelGGL(kv_decode_f16_kernel<kQ4_0>, grid, dim3(256), 0, s, (const uint8_t*)k_src,
                       (const uint8_t*)v_src, rows, (u32x4*)k_dst, (u32x4*)v_dst);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(int kv_type, const float* q, int64_t ldq, const void* k_cache, const void* v_cache,
                            int64_t n_past, int64_t t, int64_t n_head, int64_t n_kv, float scale, float* out,
                            int64_t ldo, hipStream_t s) {
  AttnArgs p;
  p.q = q;
  p.kc = (const uint8_t*)k_cache;
  p.vc = (const uint8_t*)v_cache;
  p.o = out;
  p.ldq = ldq;
  p.ldo = ldo;
  p.n_past = (int)n_past;
  p.t = (int)t;
  p.kv_len = (int)(n_past + t);
  p.n_head = (int)n_head;
  p.n_kv = (int)n_kv;
  p.group = (int)(n_head / n_kv);
  p.nqt = (int)((t + kBM - 1) / kBM);
  // log2(e) > 1, so a nonzero f32 scale never rounds to a zero factor (a
  // subnormal one is kept: the kernels run with f32 denormals), and a masked
  // score (-inf) times it stays -inf
  p.c = (float)((double)scale * 1.4426950408889634);
  const int64_t blocks = (int64_t)p.nqt * n_head;
  p.xcd = blocks % (8 * p.group) == 0 ? 1 : 0;
  // one round of workgroups (two per CU): halves; more: single halves
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const bool two = blocks <= 2 * (int64_t)cus;
  const dim3 grid((uint32_t)blocks), blk(two ? 512 : 256);
  if (kv_type != kF16 && kv_type != kQ8_0 && kv_type != kQ4_0) return hipErrorInvalidValue;
  if (two) {
    if (kv_type == kF16) hipLaunchKernelGGL((attention_kernel<kF16, 2>), grid, blk, 0, s, p);
    if (kv_type == kQ8_0) hipLaunchKernelGGL((attention_kernel<kQ8_0, 2>), grid, blk, 0, s, p);
    if (kv_type == kQ4_0) hipLaunchKernelGGL((attention_kernel<kQ4_0, 2>), grid, blk, 0, s, p);
  } else {
    if (kv_type == kF16) hipLaunchKernelGGL((attention_kernel<kF16, 1>), grid, blk, 0, s, p);
    if (kv_type == kQ8_0) hipLaunchKernelGGL((attention_kernel<kQ8_0, 1>), grid, blk, 0, s, p);
    if (kv_type == kQ4_0) hipLaunchKernelGGL((attention_kernel<kQ4_0, 1>), grid, blk, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace qp
