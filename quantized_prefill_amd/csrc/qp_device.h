// qp_device.h -- device helpers shared by the gfx950 kernels: vector types,
// loads of 2-byte-aligned block fields, and per-type decoders of one "unit"
// of 32 consecutive weights of a block.
//
// Block layouts are the GGUF / ggml on-disk convention (the pages name the
// types -- "Qwen3.5 batched prefill has no f32 dequant for IQ2_XXS, IQ3_S,
// IQ3_XXS, Q2_K", section "Cause" -- but not their bytes):
//   Q8_0  34 B / 32  : d f16 @0, qs int8[32] @2                       w = d*q
//   Q4_K 144 B / 256 : d @0, dmin @2, 12 packed 6-bit (sc, m) @4, qs[128] @16
//                      w = (d*sc)*q - dmin*m, q the nibble of qs[32*(i/64) + i%32]
//                      (low nibble for i%64 < 32), sub-block i/32
//   Q5_K 176 B / 256 : d @0, dmin @2, 12 packed (sc, m) @4, qh[32] @16, qs[128] @48
//                      w = (d*sc)*q - dmin*m, q = the Q4_K nibble | bit i/32 of qh[i%32] << 4
//   Q6_K 210 B / 256 : ql[128] @0, qh[64] @128, int8 scales[16] @192, d @208
//                      w = (d*sc[i/16])*(q-32), q = low4 | hi2 << 4
//   Q2_K  84 B / 256 : scales[16] @0 (sc low nibble, m high), qs[64] @16, d @80, dmin @82
//                      w = (d*sc)*q - dmin*m, q 2 bits of qs[32*(i/128) + i%32]
//
// A unit is weights 32u .. 32u+31 of a block (u = 0 for Q8_0, 0..7 otherwise):
// one Q8_0 block, one Q4_K sub-block, or two 16-weight scale groups of Q6_K/Q2_K.
// All products d*sc*q and dmin*m are exact in binary32 (at most 23 significant
// bits), so (d*sc)*q - dmin*m rounds once, at the subtraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

// ggml type ids (Q4_0 is a KV cache format here, not a weight type)
constexpr int kF16 = 1, kQ4_0 = 2, kQ8_0 = 8, kQ2_K = 10, kQ4_K = 12, kQ5_K = 13, kQ6_K = 14;

template <int QT> struct Fmt;
// F16 weights (one binary16 per weight) are handled by the GEMM kernels as
// blocks of 32 weights (64 bytes): K is a multiple of 256, so a row is whole
// such blocks.  The streaming dequant has its own kernel for them.
template <> struct Fmt<kF16> { static constexpr int QK = 32, TS = 64, UNITS = 1; };
template <> struct Fmt<kQ8_0> { static constexpr int QK = 32, TS = 34, UNITS = 1; };
template <> struct Fmt<kQ4_K> { static constexpr int QK = 256, TS = 144, UNITS = 8; };
template <> struct Fmt<kQ5_K> { static constexpr int QK = 256, TS = 176, UNITS = 8; };
template <> struct Fmt<kQ6_K> { static constexpr int QK = 256, TS = 210, UNITS = 8; };
template <> struct Fmt<kQ2_K> { static constexpr int QK = 256, TS = 84, UNITS = 8; };

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// nearest-even binary16 of two floats, packed low | high << 16
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  half2v h = __builtin_convertvector((float2v){lo, hi}, half2v);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// The dword that holds byte p, found by pointer arithmetic: an integer round
// trip would lose the global address space the compiler infers for kernel
// arguments and turn every load into a flat load, which also counts against
// the LDS wait counter.
__device__ __forceinline__ const uint32_t* dword_floor(const uint8_t* p) {
  return (const uint32_t*)(p - ((uintptr_t)p & 3));
}

// N dwords holding bytes [p, p + 4N) of a 2-byte-aligned address p.  Only
// 4-byte-aligned dwords that overlap [p, p + 4N) are read, so no load leaves
// the pages that hold those bytes.
template <int N>
__device__ __forceinline__ void load_dw_a2(const uint8_t* p, uint32_t (&out)[N]) {
  const uint8_t* a_p = p;
  const uintptr_t a = (uintptr_t)a_p;
  const uint32_t* base = dword_floor(a_p);
  const uint32_t sh = (uint32_t)(a & 3);  // 0 or 2
  uint32_t d[N + 1];
#pragma unroll
  for (int j = 0; j < N; ++j) d[j] = base[j];
  d[N] = base[sh ? N : N - 1];
#pragma unroll
  for (int j = 0; j < N; ++j) out[j] = __builtin_amdgcn_alignbyte(d[j + 1], d[j], sh);
}

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
  return *(const uint16_t*)p;
}

// 4 dwords from a 4-byte-aligned address, as one 16-byte load (multi-dword
// global loads need only dword alignment)
__device__ __forceinline__ void load_x4(const uint32_t* p, uint32_t* out) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  out[0] = v.x;
  out[1] = v.y;
  out[2] = v.z;
  out[3] = v.w;
}

// byte i (0..11) of three dwords s0 | s1 << 32 | s2 << 64
__device__ __forceinline__ uint32_t byte12(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t i) {
  uint32_t w = i < 4 ? s0 : (i < 8 ? s1 : s2);
  return (w >> (8 * (i & 3))) & 0xFFu;
}

// Q4_K 6-bit (scale, min) of sub-block j from the 12 packed scale bytes.
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t j,
                                              uint32_t& sc, uint32_t& m) {
  if (j < 4) {
    sc = byte12(s0, s1, s2, j) & 63u;
    m = byte12(s0, s1, s2, j + 4) & 63u;
  } else {
    const uint32_t b = byte12(s0, s1, s2, j + 4);
    sc = (b & 15u) | ((byte12(s0, s1, s2, j - 4) >> 6) << 4);
    m = (b >> 4) | ((byte12(s0, s1, s2, j) >> 6) << 4);
  }
}

// ---------------------------------------------------------------------------
// Raw fields of one unit: the quant bytes already shifted so that each byte
// holds one weight's integer code, and the per-group float factors.
//   code byte i (of 32) -> weight 32u + i
//   value_i = A[i/16] * code_i - B[i/16]    (exact products, one rounding)
// For Q8_0 the code is the signed byte; for Q6_K it is q = code - 32 with
// A = d*sc and B = 32*d*sc; Q4_K / Q2_K use A = d*sc, B = dmin*m.

struct UnitRaw {
  uint32_t code[8];  // 32 one-byte codes
  float a0, a1;      // multiplier for weights 0..15 / 16..31
  float b0, b1;      // subtrahend (0 for Q8_0)
  float sm0, sm1;    // Q4_K/Q2_K: dmin*m; Q6_K: d*sc; Q8_0: d (for the literal order)
};

// Raw<QT>: the bytes of one unit as loaded (load() issues only loads), and
// finish() turning them into a UnitRaw.  Splitting the two lets a caller keep
// the loads of the next unit in flight while it works on the current one.
template <int QT> struct Raw;

// F16 weights: the unit's 32 binary16 values, already the MFMA operand.
template <> struct Raw<kF16> {
  u32x4 v[4];
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t) {
    const u32x4* q = (const u32x4*)blk;  // rows are 512-byte multiples from a 16-byte-aligned base
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = q[i];
  }
  __device__ __forceinline__ void halves(uint32_t (&out)[16]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[4 * i] = v[i].x;
      out[4 * i + 1] = v[i].y;
      out[4 * i + 2] = v[i].z;
      out[4 * i + 3] = v[i].w;
    }
  }
};

template <> struct Raw<kQ8_0> {
  uint32_t d16, w[9], sh;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t) {
    d16 = load_u16(blk);
    const uint8_t* a_p = blk + 2;
    const uintptr_t a = (uintptr_t)a_p;
    const uint32_t* base = dword_floor(a_p);
    sh = (uint32_t)(a & 3);
    load_x4(base, w);
    load_x4(base + 4, w + 4);
    w[8] = base[sh ? 8 : 7];
  }
  __device__ __forceinline__ void finish(UnitRaw& r) const {
    const float d = f16_to_f32(d16);
#pragma unroll
    for (int j = 0; j < 8; ++j) r.code[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], sh);
    r.a0 = r.a1 = d;
    r.b0 = r.b1 = 0.f;
    r.sm0 = r.sm1 = d;
  }
};

template <> struct Raw<kQ4_K> {
  u32x4 hdr, q0, q1;
  uint32_t u;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t u_) {
    u = u_;
    hdr = *(const u32x4*)blk;  // 144-byte blocks keep 16-byte alignment
    const u32x4* qs = (const u32x4*)(blk + 16 + 32 * (u_ >> 1));
    q0 = qs[0];
    q1 = qs[1];
  }
  __device__ __forceinline__ void finish(UnitRaw& r) const {
    const float d = f16_to_f32(hdr.x & 0xFFFFu), dmin = f16_to_f32(hdr.x >> 16);
    uint32_t sc, m;
    q4k_scale_min(hdr.y, hdr.z, hdr.w, u, sc, m);
    const uint32_t sh = 4 * (u & 1);
    const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) r.code[j] = (qq[j] >> sh) & 0x0F0F0F0Fu;
    const float dsc = __fmul_rn(d, (float)sc);
    const float dm = __fmul_rn(dmin, (float)m);
    r.a0 = r.a1 = dsc;
    r.b0 = r.b1 = dm;
    r.sm0 = r.sm1 = dm;
  }
};

// Q5_K: the code of a weight is its Q4_K nibble plus the fifth bit, which for
// all 32 weights of unit u is bit u of their qh bytes (qh byte l serves weight
// l of every unit).
template <> struct Raw<kQ5_K> {
  u32x4 hdr, h0, h1, q0, q1;
  uint32_t u;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t u_) {
    u = u_;
    hdr = *(const u32x4*)blk;  // 176-byte blocks keep 16-byte alignment
    h0 = *(const u32x4*)(blk + 16);
    h1 = *(const u32x4*)(blk + 32);
    const u32x4* qs = (const u32x4*)(blk + 48 + 32 * (u_ >> 1));
    q0 = qs[0];
    q1 = qs[1];
  }
  __device__ __forceinline__ void finish(UnitRaw& r) const {
    const float d = f16_to_f32(hdr.x & 0xFFFFu), dmin = f16_to_f32(hdr.x >> 16);
    uint32_t sc, m;
    q4k_scale_min(hdr.y, hdr.z, hdr.w, u, sc, m);
    const uint32_t sh = 4 * (u & 1);
    const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const uint32_t hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) r.code[j] = ((qq[j] >> sh) & 0x0F0F0F0Fu) | (((hh[j] >> u) & 0x01010101u) << 4);
    const float dsc = __fmul_rn(d, (float)sc);
    const float dm = __fmul_rn(dmin, (float)m);
    r.a0 = r.a1 = dsc;
    r.b0 = r.b1 = dm;
    r.sm0 = r.sm1 = dm;
  }
};

template <> struct Raw<kQ6_K> {
  uint32_t ql[9], qh[9], shl_a, shh_a, scp, d16, u;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t u_) {
    u = u_;
    const uint32_t h = u_ >> 2, q4 = u_ & 3;
    const uint8_t* al_p = blk + 64 * h + 32 * (q4 & 1);
    const uintptr_t al = (uintptr_t)al_p;
    const uint8_t* ah_p = blk + 128 + 32 * h;
    const uintptr_t ah = (uintptr_t)ah_p;
    const uint32_t* bl = dword_floor(al_p);
    const uint32_t* bh = dword_floor(ah_p);
    shl_a = (uint32_t)(al & 3);
    shh_a = (uint32_t)(ah & 3);
    load_x4(bl, ql);
    load_x4(bl + 4, ql + 4);
    ql[8] = bl[shl_a ? 8 : 7];
    load_x4(bh, qh);
    load_x4(bh + 4, qh + 4);
    qh[8] = bh[shh_a ? 8 : 7];
    scp = load_u16(blk + 192 + 2 * u_);
    d16 = load_u16(blk + 208);
  }
  __device__ __forceinline__ void finish(UnitRaw& r) const {
    const uint32_t q4 = u & 3;
    const uint32_t shl = 4 * (q4 >> 1), shh = 2 * q4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t l = __builtin_amdgcn_alignbyte(ql[j + 1], ql[j], shl_a);
      const uint32_t h = __builtin_amdgcn_alignbyte(qh[j + 1], qh[j], shh_a);
      r.code[j] = ((l >> shl) & 0x0F0F0F0Fu) | (((h >> shh) & 0x03030303u) << 4);
    }
    const float d = f16_to_f32(d16);
    const float a0 = __fmul_rn(d, (float)(int8_t)(scp & 0xFFu));
    const float a1 = __fmul_rn(d, (float)(int8_t)(scp >> 8));
    r.a0 = a0;
    r.a1 = a1;
    r.b0 = __fmul_rn(a0, 32.f);
    r.b1 = __fmul_rn(a1, 32.f);
    r.sm0 = a0;
    r.sm1 = a1;
  }
};

template <> struct Raw<kQ2_K> {
  uint32_t qs[8], scp, dd, u;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t u_) {
    u = u_;
    const uint32_t* q = (const uint32_t*)(blk + 16 + 32 * (u_ >> 2));  // 84-byte blocks keep 4-byte alignment
    load_x4(q, qs);
    load_x4(q + 4, qs + 4);
    scp = load_u16(blk + 2 * u_);
    dd = *(const uint32_t*)(blk + 80);
  }
  __device__ __forceinline__ void finish(UnitRaw& r) const {
    const uint32_t sh = 2 * (u & 3);
#pragma unroll
    for (int k = 0; k < 8; ++k) r.code[k] = (qs[k] >> sh) & 0x03030303u;
    const float d = f16_to_f32(dd & 0xFFFFu), dmin = f16_to_f32(dd >> 16);
    const uint32_t s0 = scp & 0xFFu, s1 = scp >> 8;
    r.a0 = __fmul_rn(d, (float)(s0 & 15u));
    r.a1 = __fmul_rn(d, (float)(s1 & 15u));
    r.b0 = __fmul_rn(dmin, (float)(s0 >> 4));
    r.b1 = __fmul_rn(dmin, (float)(s1 >> 4));
    r.sm0 = r.b0;
    r.sm1 = r.b1;
  }
};

template <int QT> __device__ __forceinline__ void load_unit(const uint8_t* blk, uint32_t u, UnitRaw& r) {
  Raw<QT> raw;
  raw.load(blk, u);
  raw.finish(r);
}

// Span<QT, V>: V consecutive weights (V = 4 or 8, i0 % V == 0) of one block,
// loaded with a handful of coalescible loads (load) and turned into their
// exact f32 values in the literal order of the definition (value).  Used by
// the streaming dequant, whose lanes each own V consecutive outputs.
template <int QT, int V> struct Span;

template <int V> struct Span<kQ8_0, V> {
  static constexpr int N = V / 4;
  uint32_t d16, w[N + 1], sh;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t i0) {
    d16 = load_u16(blk);
    const uint8_t* a_p = blk + 2 + i0;
    const uintptr_t a = (uintptr_t)a_p;
    const uint32_t* base = dword_floor(a_p);
    sh = (uint32_t)(a & 3);
#pragma unroll
    for (int j = 0; j < N; ++j) w[j] = base[j];
    w[N] = base[sh ? N : N - 1];
  }
  __device__ __forceinline__ float value(int i) const {
    const uint32_t dw = __builtin_amdgcn_alignbyte(w[i / 4 + 1], w[i / 4], sh);
    return __fmul_rn(f16_to_f32(d16), (float)(int8_t)((dw >> (8 * (i & 3))) & 0xFFu));
  }
};

template <int V> struct Span<kQ4_K, V> {
  static constexpr int N = V / 4;
  u32x4 hdr;
  uint32_t q[N], j;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t i0) {
    hdr = *(const u32x4*)blk;
    j = i0 / 32;
    const uint32_t* qs = (const uint32_t*)(blk + 16 + 32 * (i0 / 64) + (i0 % 32));
#pragma unroll
    for (int k = 0; k < N; ++k) q[k] = qs[k];
  }
  __device__ __forceinline__ float value(int i) const {
    uint32_t sc, m;
    q4k_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
    const uint32_t code = (q[i / 4] >> (8 * (i & 3) + 4 * (j & 1))) & 15u;
    const float dsc = __fmul_rn(f16_to_f32(hdr.x & 0xFFFFu), (float)sc);
    const float dm = __fmul_rn(f16_to_f32(hdr.x >> 16), (float)m);
    return __fsub_rn(__fmul_rn(dsc, (float)code), dm);
  }
};

template <int V> struct Span<kQ5_K, V> {
  static constexpr int N = V / 4;
  u32x4 hdr;
  uint32_t q[N], h[N], j;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t i0) {
    hdr = *(const u32x4*)blk;
    j = i0 / 32;
    const uint32_t* qs = (const uint32_t*)(blk + 48 + 32 * (i0 / 64) + (i0 % 32));
    const uint32_t* qh = (const uint32_t*)(blk + 16 + (i0 % 32));
#pragma unroll
    for (int k = 0; k < N; ++k) {
      q[k] = qs[k];
      h[k] = qh[k];
    }
  }
  __device__ __forceinline__ float value(int i) const {
    uint32_t sc, m;
    q4k_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
    const uint32_t b = 8 * (i & 3);
    const uint32_t code = ((q[i / 4] >> (b + 4 * (j & 1))) & 15u) | (((h[i / 4] >> (b + j)) & 1u) << 4);
    const float dsc = __fmul_rn(f16_to_f32(hdr.x & 0xFFFFu), (float)sc);
    const float dm = __fmul_rn(f16_to_f32(hdr.x >> 16), (float)m);
    return __fsub_rn(__fmul_rn(dsc, (float)code), dm);
  }
};

template <int V> struct Span<kQ6_K, V> {
  static constexpr int N = V / 4;
  uint32_t ql[N + 1], qh[N + 1], sl, sh_, scw, d16, shl, shh;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t i0) {
    const uint32_t h = i0 / 128, r = i0 % 128, c = r / 32, l = r % 32;
    const uint8_t* al_p = blk + 64 * h + 32 * (c & 1) + l;
    const uintptr_t al = (uintptr_t)al_p;
    const uint8_t* ah_p = blk + 128 + 32 * h + l;
    const uintptr_t ah = (uintptr_t)ah_p;
    const uint32_t* bl = dword_floor(al_p);
    const uint32_t* bh = dword_floor(ah_p);
    sl = (uint32_t)(al & 3);
    sh_ = (uint32_t)(ah & 3);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      ql[k] = bl[k];
      qh[k] = bh[k];
    }
    ql[N] = bl[sl ? N : N - 1];
    qh[N] = bh[sh_ ? N : N - 1];
    const uint8_t* as_p = blk + 192 + i0 / 16;
    const uintptr_t as = (uintptr_t)as_p;
    scw = (*dword_floor(as_p)) >> (8 * (uint32_t)(as & 3));
    d16 = load_u16(blk + 208);
    shl = 4 * (c >> 1);
    shh = 2 * c;
  }
  __device__ __forceinline__ float value(int i) const {
    const uint32_t lw = __builtin_amdgcn_alignbyte(ql[i / 4 + 1], ql[i / 4], sl);
    const uint32_t hw = __builtin_amdgcn_alignbyte(qh[i / 4 + 1], qh[i / 4], sh_);
    const uint32_t b = 8 * (i & 3);
    const int q = (int)((((lw >> b) >> shl) & 15u) | ((((hw >> b) >> shh) & 3u) << 4)) - 32;
    const float dsc = __fmul_rn(f16_to_f32(d16), (float)(int8_t)(scw & 0xFFu));
    return __fmul_rn(dsc, (float)q);
  }
};

template <int V> struct Span<kQ2_K, V> {
  static constexpr int N = V / 4;
  uint32_t q[N], scw, dd, shq;
  __device__ __forceinline__ void load(const uint8_t* blk, uint32_t i0) {
    const uint32_t h = i0 / 128, j = (i0 % 128) / 32, l = i0 % 32;
    const uint32_t* qs = (const uint32_t*)(blk + 16 + 32 * h + l);
#pragma unroll
    for (int k = 0; k < N; ++k) q[k] = qs[k];
    const uint32_t so = i0 / 16;
    scw = (*(const uint32_t*)(blk + (so & ~3u))) >> (8 * (so & 3u));
    dd = *(const uint32_t*)(blk + 80);
    shq = 2 * j;
  }
  __device__ __forceinline__ float value(int i) const {
    const uint32_t code = (q[i / 4] >> (8 * (i & 3) + shq)) & 3u;
    const uint32_t s = scw & 0xFFu;
    const float dsc = __fmul_rn(f16_to_f32(dd & 0xFFFFu), (float)(s & 15u));
    const float dm = __fmul_rn(f16_to_f32(dd >> 16), (float)(s >> 4));
    return __fsub_rn(__fmul_rn(dsc, (float)code), dm);
  }
};

// Exact f32 value of weight i of the unit, in the literal left-to-right order
// of the definition (used by the bit-exact dequant).
template <int QT> __device__ __forceinline__ float unit_value_exact(const UnitRaw& r, int i) {
  const uint32_t c = (r.code[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  const bool hi = i >= 16;
  if constexpr (QT == kQ8_0) {
    return __fmul_rn(r.a0, (float)(int8_t)c);
  } else if constexpr (QT == kQ6_K) {
    // (d*sc) * (q - 32); the integer q converts exactly, keeping the sign of zero
    const float q = (float)((int)c - 32);
    return __fmul_rn(hi ? r.a1 : r.a0, q);
  } else {
    // (d*sc)*q - dmin*m
    const float p = __fmul_rn(hi ? r.a1 : r.a0, (float)c);
    return __fsub_rn(p, hi ? r.sm1 : r.sm0);
  }
}

// The same value via one fused multiply-add (identical up to the sign of a
// zero: the product is exact, so the fma rounds once, like the subtraction).
// Q8_0 codes are biased by 128 (A*(code^0x80) - 128*A) to use the unsigned
// byte converts.  Used where the result feeds a binary16 operand.
//
// Q6_K and Q8_0 (no min) take a shorter route: a byte permute turns two codes
// c into the binary16 numbers 1024 + c (exponent 10, c in the mantissa), and
// a mixed-precision fma A * (1024 + c) - (1024 + bias) * A = A * (c - bias)
// writes each binary16 result straight into its half of the output word.
// Every term is exact in f32 ((1024 + bias) * A has at most 24 significant
// bits), so the fma's only rounding is the one to binary16.
template <int QT> __device__ __forceinline__ void unit_to_f16(const UnitRaw& r, uint32_t (&out)[16]) {
  if constexpr (QT == kQ6_K || QT == kQ8_0) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    constexpr float kBias = QT == kQ6_K ? 32.f : 128.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c = r.code[j];
      if constexpr (QT == kQ8_0) c ^= 0x80808080u;  // int8 q -> q + 128
      const float a = j < 4 ? r.a0 : r.a1;
      const float cc = -__fmul_rn(a, 1024.f + kBias);
      const h2 x01 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, c, 0x07010700u));
      const h2 x23 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, c, 0x07030702u));
      const h2 r01 = {(_Float16)__builtin_fmaf(a, (float)x01[0], cc), (_Float16)__builtin_fmaf(a, (float)x01[1], cc)};
      const h2 r23 = {(_Float16)__builtin_fmaf(a, (float)x23[0], cc), (_Float16)__builtin_fmaf(a, (float)x23[1], cc)};
      out[2 * j] = __builtin_bit_cast(uint32_t, r01);
      out[2 * j + 1] = __builtin_bit_cast(uint32_t, r23);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t c = r.code[j];
    float a = j < 4 ? r.a0 : r.a1;
    float b = j < 4 ? r.b0 : r.b1;
    if constexpr (QT == kQ8_0) {
      c ^= 0x80808080u;
      b = __fmul_rn(a, 128.f);
    }
    const float v0 = __builtin_fmaf(a, (float)((c >> 0) & 0xFFu), -b);
    const float v1 = __builtin_fmaf(a, (float)((c >> 8) & 0xFFu), -b);
    const float v2 = __builtin_fmaf(a, (float)((c >> 16) & 0xFFu), -b);
    const float v3 = __builtin_fmaf(a, (float)((c >> 24) & 0xFFu), -b);
    out[2 * j] = pack_f16x2(v0, v1);
    out[2 * j + 1] = pack_f16x2(v2, v3);
  }
}

}  // namespace qp
