// gemm_wide.hip -- the dequant-on-load projection for large prefill chunks
//   Y[t, n] = sum_k X[t, k] * W[n, k]
// ("QK-norm models take the FP16 batched prefill", section "What changes":
// chunked batched prefill in FP16; the QK norm is per head).
//
// Two waves per SIMD.  A workgroup of 8 waves owns a tile of BMW = 32 MI
// tokens x BNW = 256 output features; wave w owns all BMW tokens of features
// 32 w .. 32 w + 31, i.e. MI MFMA tiles of 32 x 32 (v_mfma_f32_32x32x16_f16,
// f32 accumulators).  Each wave decodes the weights of its own features
// straight into the MFMA B-operand registers, so a weight is decoded once
// per tile and never goes through LDS as binary16, and one 16-byte LDS read
// of the activations feeds each MFMA.  The decode arithmetic (2.5-3 VALU per
// weight, about 4-5 VALU per MFMA at 256 tokens) issues beside the other
// wave's MFMAs on the same SIMD.  With K slices (KS = 2 or 4, below) the 8
// waves form KS groups over the parts of K, each owning 256 / KS features.
//
// K order.  K advances in chunks of 64 weights (4 MFMA k-steps of 16).
// Inside a chunk, k-step s takes, for lanes 0-31 (g = 0) and 32-63 (g = 1),
// the 8 weights of piece 4(s%2) + 2g + s/2 (pieces of 8).  A lane (row n,
// half g) therefore covers the two 16-weight runs [32r + 16g, 32r + 16g + 16)
// of the chunk (r = s%2), which in every K-quant layout are 16 consecutive
// code bytes of one scale group; the activations of a k-step are read from
// the same pieces.  The sum over K is the same; only its order differs.
//
// Weights.  Raw block bytes of the tile's rows are staged into LDS 128
// weights (a "step", two chunks) at a time by direct global-to-LDS dword
// loads, R rows per wave instruction (lane L copies dword L % RSD of row
// L / RSD, so consecutive rows sit RSD dwords apart, RSD odd), from a
// wave-uniform scalar offset stepping 4R rows: contiguous runs of a row per
// instruction keep the address unit cheap.  Two staging buffers: step t is
// issued two chunks before its bytes are read.
// Activations.  256-row x 64 tiles go straight from global memory into an
// LDS ring (16-byte direct loads); LDS rows keep 8 pieces of 16 B, piece p
// of row r in slot p ^ ((r >> 1) & 7), so a fragment read of 16 rows hits
// 16 distinct 16-byte bank groups.
#include <type_traits>

#include "gemm_common.h"

namespace qp {

namespace wide {

constexpr int NW = 8;               // waves per workgroup, two per SIMD
constexpr int NTW = 64 * NW;
constexpr int kLds = 160 * 1024;

// Staging of one step (128 weights) of one row.
//   NDW dwords are copied (from the dword holding the first byte of each
//   field run), RSD >= NDW is the LDS pitch (odd).  off(d, h) is the byte
//   offset from the dword-aligned block start of staged dword d for step
//   half h of a 256-weight block (before subtracting the block's start
//   misalignment, 0 or 2).
template <int QT> struct Stage;

// Q6_K half h: ql[64h, +64) (17 dwords), qh[32h, +32) (9), the 8 scales of
// the half (3), d (1).
template <> struct Stage<kQ6_K> {
  static constexpr int NDW = 30, RSD = 31, TS = 210;
  static constexpr bool P16 = false;
  static constexpr int NP = 0;
  static __device__ __forceinline__ uint32_t off(int d, int h) {
    return d < 17 ? 64 * h + 4 * d : d < 26 ? 128 + 32 * h + 4 * (d - 17) : d < 29 ? 192 + 8 * h + 4 * (d - 26) : 208;
  }
};
// Q2_K half h (blocks keep 4-byte alignment): the 8 scale bytes (2 dwords),
// qs[32h, +32) (8), d and dmin (1).
template <> struct Stage<kQ2_K> {
  static constexpr int NDW = 11, RSD = 11, TS = 84;
  static constexpr bool P16 = false;
  static constexpr int NP = 0;
  static __device__ __forceinline__ uint32_t off(int d, int h) {
    return d < 2 ? 8 * h + 4 * d : d < 10 ? 16 + 32 * h + 4 * (d - 2) : 80;
  }
};
// Q4_K half h (16-byte aligned blocks): d, dmin and the 12 scale bytes (4
// dwords), qs[64h, +64) (16).  P16: staged as NP = 5 pieces of 16 bytes,
// rows NDW dwords apart (an odd number of pieces, so the 16 rows of a
// 16-byte read land in 16 distinct bank groups); off16(j, h) is the byte
// offset of piece j within the block.
template <> struct Stage<kQ4_K> {
  static constexpr int NDW = 20, RSD = 20, TS = 144;
  static constexpr bool P16 = true;
  static constexpr int NP = 5;
  static __device__ __forceinline__ uint32_t off(int d, int h) { return d < 4 ? 4 * d : 16 + 64 * h + 4 * (d - 4); }
  static __device__ __forceinline__ uint32_t off16(int j, int h) { return j == 0 ? 0u : 16u + 64u * h + 16u * (j - 1); }
};
// Q5_K half h: header (4 dwords), qh[32] (8: every weight of the block has
// its fifth bit there), qs[64h, +64) (16).
template <> struct Stage<kQ5_K> {
  static constexpr int NDW = 28, RSD = 28, TS = 176;
  static constexpr bool P16 = true;
  static constexpr int NP = 7;
  static __device__ __forceinline__ uint32_t off(int d, int h) {
    return d < 12 ? 4 * d : 48 + 64 * h + 4 * (d - 12);
  }
  static __device__ __forceinline__ uint32_t off16(int j, int h) { return j < 3 ? 16u * j : 48u + 64u * h + 16u * (j - 3); }
};

// One decode unit: 16 weights (run r of chunk O of a step) of one row, the
// lane's k-steps r and r + 2.  read() fetches the unit's staged dwords (NU
// of them); scale() derives the unit's factors; half<H>() decodes code
// dwords 2H, 2H + 1 (8 weights) into the B operand of k-step r + 2H:
//   b[s][q]: k-step s, dword q (two binary16 weights).
struct UnitScale {
  uint32_t x, y;  // per type: two f32 factors, or two packed binary16 tables
};

// RNE16(fma(a, x, c)) for each binary16 half of x, packed as x is: one
// v_fma_mixlo_f16 and one v_fma_mixhi_f16 (the compiler would otherwise round
// through f32 pairs and a separate pack)
__device__ __forceinline__ uint32_t fma_mix_pair(float a, uint32_t x, float c) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
      : "=&v"(r)
      : "v"(a), "v"(x), "v"(c));
  return r;
}

template <int QT> struct Dec;

template <> struct Dec<kQ6_K> {
  static constexpr int NU = 13;
  // ql run r: staged dwords 8r + 4g .. + 4; qh: 17 + 4g .. + 4; the chunk's
  // scales 26 + O .. 27 + O; d 29 (each run starts delta bytes into its dword)
  template <int O, int r>
  static __device__ __forceinline__ void read(const uint32_t* row, int g, uint32_t (&u)[NU]) {
#pragma unroll
    for (int i = 0; i < 5; ++i) u[i] = row[8 * r + 4 * g + i];
#pragma unroll
    for (int i = 0; i < 5; ++i) u[5 + i] = row[17 + 4 * g + i];
    u[10] = row[26 + O];
    u[11] = row[27 + O];
    u[12] = row[29];
  }
  // a = d * sc times 2^24 and -32 d sc (both exact in f32)
  template <int O, int r>
  static __device__ __forceinline__ UnitScale scale(const uint32_t (&u)[NU], uint32_t delta, int g) {
    const float d = f16_to_f32((u[12] >> (8 * delta)) & 0xFFFFu);
    const uint32_t scw = __builtin_amdgcn_alignbyte(u[11], u[10], delta);  // the chunk's 4 scales
    const float a = __fmul_rn(d, (float)(int)(int8_t)((scw >> (8 * (g + 2 * r))) & 0xFFu));
    return {__builtin_bit_cast(uint32_t, __fmul_rn(a, 16777216.f)), __builtin_bit_cast(uint32_t, __fmul_rn(a, -32.f))};
  }
  // 6-bit codes of the four weights in staged dword j of the run (bits 0..5 of each byte)
  template <int O, int r>
  static __device__ __forceinline__ uint32_t codes(const uint32_t (&u)[NU], int j) {
    constexpr int c6 = 2 * O + r;  // which 2-bit field of qh
    const uint32_t ql = u[j], qh = u[5 + j];
    const uint32_t lo = (O ? ql >> 4 : ql) & 0x0F0F0F0Fu;
    // the 2-bit field c6 of each qh byte moved to bits 4..5
    const uint32_t hs = c6 < 2 ? qh << (4 - 2 * c6) : (c6 == 2 ? qh : qh >> 2);
    return (hs & 0x30303030u) | lo;
  }
  // A byte permute puts each code c alone in the low byte of a binary16, the
  // subnormal c 2^-24, starting delta bytes into the run; a mixed-precision fma
  // (a 2^24) (c 2^-24) - 32 a = a (c - 32) is exact in f32 (at most 8 + 11 + 6
  // significant bits), so the only rounding is the one to binary16.
  template <int O, int r, int H>
  static __device__ __forceinline__ void half(const uint32_t (&u)[NU], uint32_t delta, const UnitScale& sc,
                                              uint32_t (&b)[4][4]) {
    const float a = __builtin_bit_cast(float, sc.x), cc = __builtin_bit_cast(float, sc.y);
    const uint32_t sel01 = 0x0C010C00u + delta * 0x00010001u, sel23 = 0x0C030C02u + delta * 0x00010001u;
    uint32_t cw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) cw[j] = codes<O, r>(u, 2 * H + j);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      b[r + 2 * H][2 * k] = fma_mix_pair(a, __builtin_amdgcn_perm(cw[k + 1], cw[k], sel01), cc);
      b[r + 2 * H][2 * k + 1] = fma_mix_pair(a, __builtin_amdgcn_perm(cw[k + 1], cw[k], sel23), cc);
    }
  }
};

// Q2_K: the 4 values of a scale group, RNE16(fma(A, q, -B)) for q = 0..3,
// as two packed words; each weight picks its value by byte permute
// (selector bytes 2q, 2q + 1 of its binary16).
template <> struct Dec<kQ2_K> {
  static constexpr int NU = 6;
  // qs: staged dwords 2 + 4g .. + 3 (aligned); the chunk's scales O; d, dmin 10
  template <int O, int r>
  static __device__ __forceinline__ void read(const uint32_t* row, int g, uint32_t (&u)[NU]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = row[2 + 4 * g + i];
    u[4] = row[O];
    u[5] = row[10];
  }
  template <int O, int r>
  static __device__ __forceinline__ UnitScale scale(const uint32_t (&u)[NU], uint32_t, int g) {
    const float d = f16_to_f32(u[5] & 0xFFFFu), dmin = f16_to_f32(u[5] >> 16);
    const uint32_t s = (u[4] >> (8 * (2 * r + g))) & 0xFFu;
    const float a = __fmul_rn(d, (float)(s & 15u));
    const float bb = __fmul_rn(dmin, (float)(s >> 4));
    return {pack_f16x2(__builtin_fmaf(a, 0.f, -bb), __builtin_fmaf(a, 1.f, -bb)),
            pack_f16x2(__builtin_fmaf(a, 2.f, -bb), __builtin_fmaf(a, 3.f, -bb))};
  }
  template <int O, int r, int H>
  static __device__ __forceinline__ void half(const uint32_t (&u)[NU], uint32_t, const UnitScale& sc,
                                              uint32_t (&b)[4][4]) {
    constexpr int j2 = 2 * O + r;  // 2-bit field of qs
#pragma unroll
    for (int k = 2 * H; k < 2 * H + 2; ++k) {
      // 2q in each byte, then 2q and 2q + 1 interleaved as selectors
      const uint32_t e = (j2 == 0 ? u[k] << 1 : u[k] >> (2 * j2 - 1)) & 0x06060606u;
      const uint32_t od = e | 0x01010101u;
      const uint32_t s01 = __builtin_amdgcn_perm(od, e, 0x05010400u);
      const uint32_t s23 = __builtin_amdgcn_perm(od, e, 0x07030602u);
      b[r + 2 * H][2 * (k & 1)] = __builtin_amdgcn_perm(sc.y, sc.x, s01);
      b[r + 2 * H][2 * (k & 1) + 1] = __builtin_amdgcn_perm(sc.y, sc.x, s23);
    }
  }
};

// Q4_K / Q5_K: value = RNE16((d*sc)*q - dmin*m) with the products exact in
// f32 and one rounding at the fused subtraction, then nearest-even binary16.
// A byte permute makes each code q the subnormal binary16 q 2^-24, and the
// mixed-precision fma takes a = d sc 2^24, so a q 2^-24 is the exact product.
__device__ __forceinline__ void kquant_values(uint32_t code, float a, float bb, uint32_t& w01, uint32_t& w23) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 x01 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0u, code, 0x0C010C00u));
  const h2 x23 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0u, code, 0x0C030C02u));
  w01 = pack_f16x2(__builtin_fmaf(a, (float)x01[0], -bb), __builtin_fmaf(a, (float)x01[1], -bb));
  w23 = pack_f16x2(__builtin_fmaf(a, (float)x23[0], -bb), __builtin_fmaf(a, (float)x23[1], -bb));
}

template <> struct Dec<kQ4_K> {
  static constexpr int NU = 8;
  // header 0..3; qs of chunk O: staged dwords 4 + 8O + 4g .. + 3 (both runs:
  // low nibbles for r = 0, high for r = 1)
  template <int O, int r>
  static __device__ __forceinline__ void read(const uint32_t* row, int g, uint32_t (&u)[NU]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = row[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[4 + i] = row[4 + 8 * O + 4 * g + i];
  }
  template <int O, int r>
  static __device__ __forceinline__ UnitScale scale(const uint32_t (&u)[NU], uint32_t h, int) {
    const float d = f16_to_f32(u[0] & 0xFFFFu), dmin = f16_to_f32(u[0] >> 16);
    uint32_t sc, m;
    q4k_scale_min(u[1], u[2], u[3], 4 * h + 2 * O + r, sc, m);
    return {__builtin_bit_cast(uint32_t, __fmul_rn(__fmul_rn(d, (float)sc), 16777216.f)),
            __builtin_bit_cast(uint32_t, __fmul_rn(dmin, (float)m))};
  }
  template <int O, int r, int H>
  static __device__ __forceinline__ void half(const uint32_t (&u)[NU], uint32_t, const UnitScale& sc,
                                              uint32_t (&b)[4][4]) {
#pragma unroll
    for (int k = 2 * H; k < 2 * H + 2; ++k) {
      const uint32_t code = (u[4 + k] >> (4 * r)) & 0x0F0F0F0Fu;
      kquant_values(code, __builtin_bit_cast(float, sc.x), __builtin_bit_cast(float, sc.y), b[r + 2 * H][2 * (k & 1)],
                    b[r + 2 * H][2 * (k & 1) + 1]);
    }
  }
};

template <> struct Dec<kQ5_K> {
  static constexpr int NU = 12;
  // header 0..3; qh bytes 16g .. + 15: staged dwords 4 + 4g; qs of chunk O: 12 + 8O + 4g
  template <int O, int r>
  static __device__ __forceinline__ void read(const uint32_t* row, int g, uint32_t (&u)[NU]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = row[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[4 + i] = row[4 + 4 * g + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[8 + i] = row[12 + 8 * O + 4 * g + i];
  }
  template <int O, int r>
  static __device__ __forceinline__ UnitScale scale(const uint32_t (&u)[NU], uint32_t h, int) {
    const float d = f16_to_f32(u[0] & 0xFFFFu), dmin = f16_to_f32(u[0] >> 16);
    uint32_t sc, m;
    q4k_scale_min(u[1], u[2], u[3], 4 * h + 2 * O + r, sc, m);
    return {__builtin_bit_cast(uint32_t, __fmul_rn(__fmul_rn(d, (float)sc), 16777216.f)),
            __builtin_bit_cast(uint32_t, __fmul_rn(dmin, (float)m))};
  }
  // the fifth bit of weight l is bit j = 4h + 2O + r of qh byte l
  template <int O, int r, int H>
  static __device__ __forceinline__ void half(const uint32_t (&u)[NU], uint32_t h, const UnitScale& sc,
                                              uint32_t (&b)[4][4]) {
    const uint32_t j = 4 * h + 2 * O + r;
#pragma unroll
    for (int k = 2 * H; k < 2 * H + 2; ++k) {
      const uint32_t code = ((u[8 + k] >> (4 * r)) & 0x0F0F0F0Fu) | (((u[4 + k] >> j) & 0x01010101u) << 4);
      kquant_values(code, __builtin_bit_cast(float, sc.x), __builtin_bit_cast(float, sc.y), b[r + 2 * H][2 * (k & 1)],
                    b[r + 2 * H][2 * (k & 1) + 1]);
    }
  }
};

// LDS offset (halfs) of 16-byte piece `piece` of activation row `row`
__device__ __forceinline__ int xswz(int row, int piece) { return (row * 8 + (piece ^ ((row >> 1) & 7))) * 8; }

// s_waitcnt vmcnt(N), the other counters unconstrained
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// KS: K slices.  KS = 2 or 4 splits the 8 waves into KS groups that take
// the KS parts of K with buffers of their own (a tile of 32 * MI tokens x
// 256 / KS features); the other groups' sums join the first's through LDS
// at the end, in slice order.  For short prefill chunks, where
// 256-feature tiles would leave CUs idle and a K split across workgroups
// writes partial sums to memory.
template <int QT, int MI, int KS = 1>
struct Cfg {
  static constexpr int NWS = NW / KS;                      // waves per K slice
  static constexpr int BMW = 32 * MI, BNW = 32 * NWS;
  static constexpr int RSD = Stage<QT>::RSD;
  static constexpr int R = 64 / RSD;                       // rows per staging instruction
  static constexpr int NG = (BNW + R - 1) / R;             // groups of R rows per tile
  static constexpr int NI16 = Stage<QT>::NP * BNW / 64;   // P16 types: 16-byte staging loads per tile and step
  static constexpr int NI = Stage<QT>::P16 ? (NI16 + NWS - 1) / NWS : (NG + NWS - 1) / NWS;  // per wave and step
  static constexpr int XTILE = BMW * 64;                   // halfs per activation chunk
  static constexpr int RAWB = BNW * RSD + 64;              // dwords per staging buffer (64 of padding)
  static constexpr int XB = 3;
  static constexpr int XL = BMW * 8 / 64 / NWS;            // activation loads per wave and chunk (16 B per lane)
  static_assert((NG - 1) * R * RSD + 64 <= RAWB, "the padding takes the last group's spare lanes");
  static_assert(!Stage<QT>::P16 || (NI16 * 64 == Stage<QT>::NP * BNW && RSD == 4 * Stage<QT>::NP),
                "16-byte staging: whole loads per tile, rows of NP pieces");
  static_assert(KS * (XB * XTILE * 2 + 2 * RAWB * 4) <= kLds, "LDS budget");
  static_assert(XL * NWS * 64 == BMW * 8, "whole activation loads per wave");
  static_assert((KS - 1) * NWS * MI * 16 * 64 <= XB * XTILE / 2 * KS, "the slice sums fit the activation buffers");
};

template <int QT, int MI, int KS = 1>
struct Smem {
  using C = Cfg<QT, MI, KS>;
  _Float16 x[KS][C::XB][C::XTILE];
  uint32_t raw[KS][2][C::RAWB];
};

}  // namespace wide

using namespace wide;

// Main loop and epilogue of one tile; FULL: every row of the tile is inside
// the weight tensor (staging addresses from a per-lane constant and a
// per-instruction scalar offset).
//
// Wave w owns features 32 w .. 32 w + 31 of the tile.  Its B operands sit in
// one set of four k-step slots; slot x is refilled for the next chunk in the
// k-step after the MFMAs that last read it.  A chunk's decode has two units
// (runs r = 0, 1; unit r fills k-steps r and r + 2, as halves H = 0, 1).
// Schedule of chunk c:
//   k-step 0: read the staged bytes of unit 0 of chunk c + 1; slot 3 <- unit
//             1, half 1 of chunk c
//   k-step 1: slot 0 <- unit 0, half 0 of chunk c + 1; read the staged bytes
//             of unit 1 of chunk c + 1
//   k-step 2: slot 1 <- unit 1, half 0 of chunk c + 1
//   wait for the activations of chunk c + 1 (and, for odd c, the staging of
//   the step after next); barrier
//   k-step 3: load activation chunk c + 3 into the buffer chunk c used;
//             slot 2 <- unit 0, half 1 of chunk c + 1
// In every k-step the MI MFMAs issue with one activation fragment read after
// each, for the same M block of the next k-step (k-step 0 of chunk c + 1
// after k-step 3: its activations are in place once the barrier passed).
// Staging of step t + 2 (into the buffer step t used) is issued in four
// parts, at k-step 3 of chunk 2t and k-steps 0..2 of chunk 2t + 1: every
// read of step t happens before the barrier of chunk 2t, and step t + 2 is
// first read after the barrier of chunk 2t + 2.  Indices past the end are
// clamped to the last chunk or step (the loads and decodes then repeat valid
// data that nothing uses), so the loop body has no branches.
template <int QT, int MODE, int MI, bool FULL, int KS = 1>
__device__ __forceinline__ void wide_tile(const GemmParams& p, Smem<QT, MI, KS>& sm, int n0, int m0) {
  using C = Cfg<QT, MI, KS>;
  constexpr int NWS = C::NWS;
  using S = Stage<QT>;
  using D = Dec<QT>;
  constexpr int BMW = C::BMW, BNW = C::BNW, XB = C::XB, RSD = C::RSD, R = C::R, NI = C::NI, XL = C::XL;
  // routed modes: opaque to the optimizer, so that in the loop over tiles
  // values derived from the thread index are formed per tile, not held in
  // registers across tiles
  int tid = threadIdx.x;
  if constexpr (MODE == kGrouped || MODE == kGroupedGU || MODE == kGroupedDown) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wv / NWS;      // K slice of the wave
  const int w = wv % NWS;       // wave within the slice
  const int g = lane >> 5;
  const int m_rows = min(BMW, p.t - m0);
  const int kslice = p.k / KS;  // the slice: weights kslice * ks .. of every row
  const int ub0 = ks * (kslice / 256);  // its first block
  const int nch = kslice / BK;  // chunks of 64 (a multiple of 4)
  const int nsteps = nch / 2;   // staging steps of 128
  const int64_t rb = p.rb;
  const uint32_t rb3 = (uint32_t)(rb & 3);

  // ---- activation copy: load q of wave w puts lane l at tile row
  // w * BMW / NWS + 8 q + l / 8, slot l % 8
  const _Float16* xtile = (const _Float16*)p.x + (int64_t)m0 * p.ldx + (int64_t)ks * kslice;
  uint32_t xoff[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int row = w * (BMW / NWS) + 8 * q + (lane >> 3);
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    int xr = min(row, m_rows - 1);
    if constexpr (MODE == kGrouped || MODE == kGroupedGU) xr = p.list[xr] / p.top_k;  // the token of compact row xr
    xoff[q] = (uint32_t)(2 * (xr * p.ldx + 8 * piece));
  }
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)xtile, (short)0, -1, 0x00020000);
  auto load_x = [&](int c) __attribute__((always_inline)) {
    c = min(c, nch - 1);  // past the end: the last chunk again (keeps the load count uniform)
    _Float16* dst = sm.x[ks][c % XB] + w * (BMW / NWS) * 64;
#pragma unroll
    for (int q = 0; q < XL; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (__attribute__((address_space(3))) void*)(dst + 8 * q * 64), 16,
                                               (int)xoff[q], 128 * c, 0, 0);
  };

  // ---- weight staging: row n of the tile at LDS dword RSD * n (RSD odd).
  // Instruction q of wave w stages group grp = NW q + w of R rows (past the
  // last group: the last group again, the same bytes to the same place); lane
  // L loads the dword that belongs at group dword L, i.e. dword L % RSD of row
  // grp R + L / RSD.  Every lane loads, so no branch splits the loop: lanes
  // past the group's R rows write the first dwords of the next rows, exactly
  // what those rows' own loads write there, and a lane on a row's padding
  // dword writes a copy of the row's last staged dword there.  In the last
  // group the lanes past the tile's rows copy its last row instead, into the
  // 64 dwords of padding after the buffer (rows past the tile need not exist).
  const int sgr = lane / RSD, sd = min(lane % RSD, S::NDW - 1);
  const int sgr_last = min(sgr, BNW - 1 - (C::NG - 1) * R);
  const uint8_t* wtile = p.w + (int64_t)n0 * rb;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)wtile, (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc_part =
      __builtin_amdgcn_make_buffer_rsrc((void*)wtile, (short)0, FULL ? -1 : (int)((int64_t)(p.n - n0) * rb), 0x00020000);
  // kGroupedGU: staged rows 0..127 are gate rows n0.., 128..255 the same up
  // rows; a 16-byte load lies wholly in one half (128 NP pieces = 2 NP loads)
  static_assert(MODE != kGroupedGU || (S::P16 && FULL && KS == 1 && C::NI16 % 2 == 0), "gate/up tiles: 16-byte staging");
  const __amdgpu_buffer_rsrc_t wrsrc_up =
      MODE == kGroupedGU ? __builtin_amdgcn_make_buffer_rsrc((void*)(p.w2 + (int64_t)n0 * rb), (short)0, -1, 0x00020000)
                         : wrsrc;
  // FULL: the dword-aligned start of the lane's run splits into a per-lane
  // part and a per-instruction part (rows 2 apart start at the same offset
  // within a dword, and R is even wherever rb % 4 != 0), for block offsets 0
  // and 2 mod 4 and the two step halves
  auto lane_off = [&](int gr, uint32_t& v00, uint32_t& va, uint32_t& vh) __attribute__((always_inline)) {
    v00 = (((uint32_t)(gr * rb)) & ~3u) + S::off(sd, 0);
    va = ((((uint32_t)(gr * rb) + 2u) & ~3u) - (((uint32_t)(gr * rb)) & ~3u));  // 0 or 4
    vh = S::off(sd, 1) - S::off(sd, 0);
  };
  uint32_t vo00, vo_a, vo_h, vl00, vl_a, vl_h;
  lane_off(sgr, vo00, vo_a, vo_h);
  lane_off(sgr_last, vl00, vl_a, vl_h);
  // P16 types: load q of wave w is load gi = NWS q + w of the tile (past the
  // last: the last again); lane L copies piece P = 64 gi + L of the staged
  // rows, piece P % NP of row P / NP, to LDS dword 4 P (row pitch 4 NP)
  uint32_t v16a[S::P16 ? NI : 1], v16b[S::P16 ? NI : 1];  // step halves 0 and 1
  if constexpr (S::P16) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int gi = min(NWS * q + w, C::NI16 - 1);
      const int pc = 64 * gi + lane;
      const int row = pc / S::NP, j = pc - row * S::NP;
      const int wr = MODE == kGroupedGU ? (row & 127) : row;  // the row within its tensor's tile rows
      v16a[q] = (uint32_t)(wr * rb) + S::off16(j, 0);
      v16b[q] = (uint32_t)(wr * rb) + S::off16(j, 1);
    }
  }
  // part [Q0, Q1) of the loads of step st (clamped to the last step) into buffer buf
  auto stage_part = [&](int st, int buf, auto q0c, auto q1c) __attribute__((always_inline)) {
    constexpr int Q0 = decltype(q0c)::value, Q1 = decltype(q1c)::value;
    st = min(st, nsteps - 1);
    const int u = (st >> 1) + ub0, h = st & 1;
    const uint32_t boff = (uint32_t)u * S::TS;
    uint32_t* dst = sm.raw[ks][buf];
    if constexpr (S::P16) {
      // whole 16-byte pieces; rows past the tensor (not FULL) read zeros
      // past wrsrc_part's record count, as below
#pragma unroll
      for (int q = Q0; q < Q1; ++q) {
        const int gi = min(NWS * q + w, C::NI16 - 1);
        const uint32_t v = h ? v16b[q] : v16a[q];
        if constexpr (MODE == kGroupedGU)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(2 * gi < C::NI16 ? wrsrc : wrsrc_up,
                                                   (__attribute__((address_space(3))) void*)(dst + 256 * gi), 16, (int)v,
                                                   (int)boff, 0, 0);
        else if constexpr (FULL)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (__attribute__((address_space(3))) void*)(dst + 256 * gi), 16,
                                                   (int)v, (int)boff, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc_part, (__attribute__((address_space(3))) void*)(dst + 256 * gi),
                                                   16, (int)(v + boff), 0, 0, 0);
      }
    } else if constexpr (FULL) {
      const uint32_t ab = (boff >> 1) & 1u;
      const uint32_t v0 = vo00 + ab * vo_a + (uint32_t)h * vo_h;
      const uint32_t vl = vl00 + ab * vl_a + (uint32_t)h * vl_h;
#pragma unroll
      for (int q = Q0; q < Q1; ++q) {
        const int grp = min(NWS * q + w, C::NG - 1);
        const bool last = NWS * q + NWS - 1 >= C::NG - 1 && grp == C::NG - 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (__attribute__((address_space(3))) void*)(dst + grp * R * RSD), 4,
                                                 (int)(last ? vl : v0), (int)((int64_t)grp * R * rb + (boff & ~3u)), 0, 0);
      }
    } else {
      // the tile's last rows lie past the tensor: the whole offset goes in
      // the range-checked per-lane offset, and loads at or past the tensor's
      // end (wrsrc_part's record count) return zeros, which only rows past
      // the tensor receive (their outputs are not stored)
      const uint32_t v0 = ((((uint32_t)(sgr * rb) + boff) & ~3u) + S::off(sd, h));
#pragma unroll
      for (int q = Q0; q < Q1; ++q) {
        const int grp = min(NWS * q + w, C::NG - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc_part,
                                                 (__attribute__((address_space(3))) void*)(dst + grp * R * RSD), 4,
                                                 (int)(v0 + (uint32_t)(grp * R * rb)), 0, 0, 0);
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, NI / 4>;
  using P2 = std::integral_constant<int, NI / 2>;
  using P3 = std::integral_constant<int, 3 * NI / 4>;
  using P4 = std::integral_constant<int, NI>;

  // ---- decode side: the lane's row is tile row 32 w + l % 32 (kGroupedGU:
  // lanes l % 32 < 16 gate row 16 w + l % 16, the others the same up row)
  const int nrow = MODE == kGroupedGU ? ((lane & 16) << 3) + 16 * w + (lane & 15) : 32 * w + (lane & 31);
  const uint32_t rdelta = (uint32_t)((FULL ? nrow : min(nrow, p.n - 1 - n0)) & 1) * rb3;  // 2: row starts 2 bytes into a dword
  // staged bytes of unit (O, r) of step st (clamped)
  auto read_unit = [&](int st, auto oc, auto rc, uint32_t (&u)[D::NU]) __attribute__((always_inline)) {
    st = min(st, nsteps - 1);
    D::template read<decltype(oc)::value, decltype(rc)::value>(sm.raw[ks][st & 1] + nrow * RSD, g, u);
  };
  // Q6_K: misalignment of the block start; Q4_K / Q5_K: the step's half
  auto dec_arg = [&](int st) __attribute__((always_inline)) -> uint32_t {
    st = min(st, nsteps - 1);
    if constexpr (QT == kQ6_K)
      return (rdelta + (uint32_t)((st >> 1) + ub0) * S::TS) & 3;
    else
      return (uint32_t)(st & 1);
  };

  float16v acc[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) acc[i] = (float16v){};
  // The loop over K for the first MA M blocks (a tile of at most 32 MA rows
  // skips the MFMAs and fragment reads of the blocks past its rows; MA = 4,
  // 6 or 8 for 256-row tiles).
  auto main_loop = [&](auto mac) __attribute__((always_inline)) {
    constexpr int MA = decltype(mac)::value;
    // activation fragment of k-step s: row 32 i + l % 32, piece 4 (s % 2) + 2 g + s / 2;
    // rows 32 apart share the slot order
    int aoff[4];
  #pragma unroll
    for (int s = 0; s < 4; ++s) aoff[s] = 2 * xswz(lane & 31, 4 * (s & 1) + 2 * g + (s >> 1));
    auto a_ptr = [&](int c, int s) __attribute__((always_inline)) -> const char* {
      return (const char*)sm.x[ks][min(c, nch - 1) % XB] + aoff[s];
    };

    uint32_t b[4][4];
    half8 a[MA];
    uint32_t u0[D::NU], u1[D::NU];
    UnitScale s0, s1;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // ---- prologue: steps 0 and 1 staged, activation chunks 0 .. 2; chunk 0's
    // slots 0..2 decoded (slot 3 in the loop's first k-step).  Only step 0
    // and chunk 0 are waited for here (issued first); step 1 and chunk 1 land
    // by chunk 0's barrier, whose wait leaves only chunk 2 in flight.
    stage_part(0, 0, P0{}, P4{});
    load_x(0);
    stage_part(1, 1, P0{}, P4{});
    load_x(1);
    load_x(2);
    wait_vm<NI + 2 * XL>();
    lds_barrier();
    {
      const char* ap = a_ptr(0, 0);
  #pragma unroll
      for (int i = 0; i < MA; ++i) a[i] = *(const half8*)(ap + 32 * 64 * 2 * i);
    }
    read_unit(0, I0{}, I0{}, u0);
    read_unit(0, I0{}, I1{}, u1);
    s0 = D::template scale<0, 0>(u0, dec_arg(0), g);
    s1 = D::template scale<0, 1>(u1, dec_arg(0), g);
    D::template half<0, 0, 0>(u0, dec_arg(0), s0, b);
    D::template half<0, 1, 0>(u1, dec_arg(0), s1, b);
    D::template half<0, 0, 1>(u0, dec_arg(0), s0, b);

    // k-step s of chunk c: MFMA i, then the read of M block i of the next
    // fragment (k-step s + 1, or k-step 0 of chunk c + 1)
    auto mfmas = [&](int c, int s) __attribute__((always_inline)) {
      const char* ap = s < 3 ? a_ptr(c, s + 1) : a_ptr(c + 1, 0);
  #pragma unroll
      for (int i = 0; i < MA; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], __builtin_bit_cast(half8, b[s]), acc[i], 0, 0, 0);
        a[i] = *(const half8*)(ap + 32 * 64 * 2 * i);
      }
    };
    // per MFMA: the fragment read after it, a share of the VALU and of the global loads
    auto interleave = [&](auto nvc, auto nmc) __attribute__((always_inline)) {
      constexpr int NV = decltype(nvc)::value, NM = decltype(nmc)::value;
  #pragma unroll
      for (int i = 0; i < MA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x020, (NM + MA - 1) / MA, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x002, (NV + MA - 1) / MA, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using V0 = std::integral_constant<int, 40>;

    // chunk c = 2 st + O
    auto chunk = [&](int st, auto oc) __attribute__((always_inline)) {
      constexpr int O = decltype(oc)::value;
      constexpr int ON = 1 - O;  // chunk c + 1 within its step
      const int c = 2 * st + O;
      const int sn = O ? st + 1 : st;  // step of chunk c + 1
      using ONc = std::integral_constant<int, ON>;
      const uint32_t da = dec_arg(st), dn = dec_arg(sn);
      // k-step 0
      if constexpr (O == 1) stage_part(st + 2, st & 1, P1{}, P2{});
      mfmas(c, 0);
      D::template half<O, 1, 1>(u1, da, s1, b);  // slot 3, this chunk
      read_unit(sn, ONc{}, I0{}, u0);
      interleave(V0{}, std::integral_constant<int, O == 1 ? P2::value - P1::value : 0>{});
      // k-step 1
      if constexpr (O == 1) stage_part(st + 2, st & 1, P2{}, P3{});
      mfmas(c, 1);
      s0 = D::template scale<ON, 0>(u0, dn, g);
      D::template half<ON, 0, 0>(u0, dn, s0, b);  // slot 0, next chunk
      read_unit(sn, ONc{}, I1{}, u1);
      interleave(V0{}, std::integral_constant<int, O == 1 ? P3::value - P2::value : 0>{});
      // k-step 2
      if constexpr (O == 1) stage_part(st + 2, st & 1, P3{}, P4{});
      mfmas(c, 2);
      s1 = D::template scale<ON, 1>(u1, dn, g);
      D::template half<ON, 1, 0>(u1, dn, s1, b);  // slot 1, next chunk
      interleave(V0{}, std::integral_constant<int, O == 1 ? P4::value - P3::value : 0>{});
      // activations of chunk c + 1 (and for odd c the staging of step st + 2) have landed
      if constexpr (O == 1)
        wait_vm<XL + NI>();
      else
        wait_vm<XL>();
      lds_barrier();
      // k-step 3
      load_x(c + 3);  // its buffer held chunk c
      if constexpr (O == 0) stage_part(st + 2, st & 1, P0{}, P1{});  // its buffer held step st
      mfmas(c, 3);
      D::template half<ON, 0, 1>(u0, dn, s0, b);  // slot 2, next chunk
      interleave(V0{}, std::integral_constant<int, XL + (O == 0 ? P1::value : 0)>{});
    };

    for (int st = 0; st < nsteps; ++st) {
      chunk(st, I0{});
      chunk(st, I1{});
    }
  };
  if constexpr (MI == 8) {
    if (m_rows <= 128)
      main_loop(std::integral_constant<int, 4>{});
    else if (m_rows <= 192)
      main_loop(std::integral_constant<int, 6>{});
    else
      main_loop(std::integral_constant<int, 8>{});
  } else {
    main_loop(std::integral_constant<int, MI>{});
  }
  // routed down pass: the tile's output rows (pairs list[r]) go through LDS,
  // loaded once here instead of one dependent load per store below
  int out_row = 0;
  if constexpr (MODE == kGroupedDown) {
    if (tid < BMW) out_row = p.list[min(tid, m_rows - 1)];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped re-loads past the end have landed
  lds_barrier();
  if constexpr (MODE == kGroupedDown) {  // the staging buffers are free now
    if (tid < BMW) ((int*)sm.raw[0][0])[tid] = out_row;
    lds_barrier();
  }
  if constexpr (KS > 1) {
    // the other slices' sums into the first's, in slice order (one dword
    // per lane and value), then all past a barrier before the stores reuse
    // the buffer
    float* red = (float*)&sm.x[0][0][0] + lane;
    constexpr int SW = MI * 16 * 64;  // floats per wave
    if (ks > 0) {
      float* dst = red + ((ks - 1) * NWS + w) * SW;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int a = 0; a < 16; ++a) dst[(16 * i + a) * 64] = acc[i][a];
    }
    lds_barrier();
    if (ks == 0) {
#pragma unroll
      for (int k = 1; k < KS; ++k) {
        const float* src = red + ((k - 1) * NWS + w) * SW;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int a = 0; a < 16; ++a) acc[i][a] = acc[i][a] + src[(16 * i + a) * 64];
      }
    }
    lds_barrier();
    if (ks > 0) return;
  }

  // ---- epilogue: 16-byte stores through a per-wave LDS transpose
  float* scr = (float*)sm.x + 32 * 40 * w;
  if constexpr (MODE == kGroupedGU) {
    // column l % 32 of a block is gate feature n0 + 16 w + l % 16 for l % 32
    // < 16, else the same up feature, over the same tokens: lanes l and
    // l ^ 16 trade one value per pair of accumulators, the lane with the gate
    // value forms h = SiLU(g) u = g u / (1 + 2^(-g log2 e)) for the even one,
    // its partner for the odd one (row + 1).  Stores through a buffer whose
    // record count ends at the tile's last row: rows past it are dropped.
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const bool up = (ln & 16) != 0;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.y, (short)0, (int)((int64_t)m_rows * p.ldy * 4), 0x00020000);
    const uint32_t voff = (uint32_t)(((4 * (ln >> 5) + (up ? 1 : 0)) * p.ldy + n0 + 16 * w + (ln & 15)) * 4);
    const uint32_t rstep = (uint32_t)(p.ldy * 4);
    // a bit mask (opaque to the optimizer, which would otherwise turn the
    // choice between two accumulators into a run-time register index)
    uint32_t upm = up ? ~0u : 0u;
    asm volatile("" : "+v"(upm));
    auto pick = [&](float x_up, float x_gate) __attribute__((always_inline)) {
      return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x_up) & upm) |
                                           (__builtin_bit_cast(uint32_t, x_gate) & ~upm));
    };
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int a = 0; a < 16; a += 2) {
        const float recv = __shfl_xor(pick(acc[i][a], acc[i][a + 1]), 16, 64);
        const float gv = pick(recv, acc[i][a]);
        const float uv = pick(acc[i][a + 1], recv);
        const float h = gv * uv * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(gv * -1.44269504088896341f));
        const uint32_t row = (uint32_t)(32 * i + 8 * (a >> 2) + (a & 3));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, h), yr, (int)(voff + row * rstep), 0, 0);
      }
    return;
  }
  float16v accs[MI][1];
#pragma unroll
  for (int i = 0; i < MI; ++i) accs[i][0] = acc[i];
  if constexpr (MODE == kGroupedDown) {
    // routed down pass: row r of the tile is pair list[r]'s row of y
    store_tiles_vec<MI, 1>(accs, m_rows, n0 + 32 * w, p.n, lane, scr,
                           [&](int r) __attribute__((always_inline)) {
                             return p.y + (int64_t)((const int*)sm.raw[0][0])[r] * p.ldy;  // rows past the tile: not stored
                           });
  } else {
    store_tiles_vec<MI, 1>(accs, m_rows, n0 + 32 * w, p.n, lane, scr,
                           [&](int r) __attribute__((always_inline)) { return p.y + (int64_t)(m0 + r) * p.ldy; });
  }
}

// Routed modes whose workgroups loop over tiles (one workgroup per CU): the
// types whose loop fits the register budget without spills; the others run
// one tile per workgroup.
constexpr bool wide_persistent(int qt, int mode) {
  return mode == kGroupedGU || qt == kQ4_K || qt == kQ2_K;
}

// Routed modes: linear tile b of pk.tcols x (table length, a multiple of 8)
// is table tile b % 8 + 8 ((b / 8) / tcols), column tile (b / 8) % tcols.
// Returns false for an entry past the table (no rows; nothing touched).
template <int QT, int MODE, int MI, int KS>
__device__ __forceinline__ bool routed_tile(const GemmParams& pk, Smem<QT, MI, KS>& sm, uint32_t b) {
  const uint32_t kx = b >> 3;
  const int ti = (int)((b & 7) + 8 * (kx / (uint32_t)pk.tcols));
  int tile_x = (int)(kx % (uint32_t)pk.tcols);
  const u32x4 te = *(const u32x4*)(pk.tiles + 4 * ti);
  if (te[2] == 0) return false;  // past the table's tiles
  const int e = (int)te[0], base = (int)te[3];  // expert, first compact row of the tile
  GemmParams p = pk;
  p.t = (int)te[2];          // the tile's rows
  p.list = pk.list + base;  // the tile's pairs
  if constexpr (MODE == kGroupedGU) {
    // gate/up with SiLU: the column tile is 128 features of h (gate and up
    // rows of one expert)
    p.w = pk.w + (int64_t)e * pk.estride;
    p.w2 = pk.w2 + (int64_t)e * pk.estride;
    p.y = pk.y + (int64_t)base * pk.ldy;
    wide_tile<QT, MODE, MI, true, KS>(p, sm, tile_x * 128, 0);
  } else {
    // the column tile picks the segment (gate / up, or the down projection)
    int sg = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i) sg += (i < pk.seg.nseg && tile_x >= pk.seg.tile0[i]);
    tile_x -= pk.seg.tile0[sg];
    p.w = pk.seg.w[sg] + (int64_t)e * pk.estride;
    p.n = pk.seg.n[sg];
    p.ldy = pk.seg.ldy[sg];
    if constexpr (MODE == kGrouped) {  // gate / up: X rows are the pairs' tokens, y the compact rows
      p.y = pk.seg.y[sg] + (int64_t)base * pk.seg.ldy[sg];
    } else {                           // down: A the compact rows, y the pairs' rows
      p.x = (const _Float16*)pk.x + (int64_t)base * pk.ldx;
      p.y = pk.seg.y[sg];
    }
    // every column tile is whole: the launcher takes segments of whole tiles only
    wide_tile<QT, MODE, MI, true, KS>(p, sm, tile_x * Cfg<QT, MI, KS>::BNW, 0);
  }
  return true;
}

// Grid: (column tiles, token tiles).  kMulti: projections over one X, each
// a segment of whole column tiles (its own weights, rows and output).
// Routed modes: gridDim.x workgroups (a multiple of 8) run linear tiles g,
// g + gridDim.x, ... in turn (see routed_tile).  Workgroups go to the 8 XCDs
// in turn (g % 8), and so does every tile of a workgroup: an XCD runs whole
// table tiles, all their column tiles one after the other, and the tile's
// activation rows are fetched into its L2 once rather than by every XCD.
template <int QT, int MODE, int MI, int KS = 1>
__global__ __launch_bounds__(NTW) void gemm_wide_kernel(GemmParams pk) {
  __shared__ __attribute__((aligned(16))) Smem<QT, MI, KS> sm;
  if constexpr (MODE == kGrouped || MODE == kGroupedGU || MODE == kGroupedDown) {
    if constexpr (wide_persistent(QT, MODE)) {
      const uint32_t total = (uint32_t)pk.tcols * (uint32_t)pk.t;
      for (uint32_t b = blockIdx.x; b < total; b += gridDim.x)
        if (routed_tile<QT, MODE, MI, KS>(pk, sm, b)) __syncthreads();  // the epilogue's LDS, before the next staging
    } else {
      routed_tile<QT, MODE, MI, KS>(pk, sm, blockIdx.x);
    }
  } else {
    GemmParams p = pk;
    int tile_x = blockIdx.x;
    if constexpr (MODE == kMulti) {
      int sg = 0;
#pragma unroll
      for (int i = 1; i < kMaxSeg; ++i) sg += (i < pk.seg.nseg && tile_x >= pk.seg.tile0[i]);
      tile_x -= pk.seg.tile0[sg];
      p.w = pk.seg.w[sg];
      p.n = pk.seg.n[sg];
      p.k = pk.seg.k[sg];  // a K part: its weights start at seg.w, its activations xoff into each row
      p.x = (const _Float16*)pk.x + pk.seg.xoff[sg];
      p.y = pk.seg.y[sg];
      p.ldy = pk.seg.ldy[sg];
    }
    const int m0 = blockIdx.y * Cfg<QT, MI>::BMW;
    const int n0 = tile_x * Cfg<QT, MI, KS>::BNW;
    if (n0 + Cfg<QT, MI, KS>::BNW <= p.n)
      wide_tile<QT, MODE, MI, true, KS>(p, sm, n0, m0);
    else
      wide_tile<QT, MODE, MI, false, KS>(p, sm, n0, m0);
  }
}

bool wide_supported(int qtype, int mode) {
  if (mode == kGroupedGU) return qtype == kQ4_K || qtype == kQ5_K;
  return (qtype == kQ6_K || qtype == kQ2_K || qtype == kQ4_K || qtype == kQ5_K) &&
         (mode == kPlainF16 || mode == kMulti || mode == kGrouped || mode == kGroupedDown);
}

int wide_cols() { return 32 * NW; }

template <int QT, int MODE, int MI>
static void launch_wide_t(const GemmParams& p, uint32_t col_tiles, hipStream_t s) {
  constexpr int BMW = 32 * MI;
  if constexpr (MODE == kGrouped || MODE == kGroupedGU || MODE == kGroupedDown) {
    // p.t carries the size of the tile table (its largest possible length, a
    // multiple of 8)
    // persistent types: one workgroup per CU (a multiple of 8), or fewer for
    // a smaller table; the others one workgroup per tile
    GemmParams q = p;
    q.tcols = (int)col_tiles;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
      cus = 256;
    const uint32_t total = col_tiles * (uint32_t)p.t;
    const uint32_t g = wide_persistent(QT, MODE) ? std::min(total, (uint32_t)(cus / 8 * 8)) : total;
    hipLaunchKernelGGL((gemm_wide_kernel<QT, MODE, MI>), dim3(g), dim3(NTW), 0, s, q);
  } else {
    const dim3 grid(col_tiles, (uint32_t)((p.t + BMW - 1) / BMW));
    hipLaunchKernelGGL((gemm_wide_kernel<QT, MODE, MI>), grid, dim3(NTW), 0, s, p);
  }
}

// Tiles of 32 * mi tokens x 256 features (mi = 8 or 4); kMulti: p.seg
// holds the segments and col_tiles their total.
hipError_t launch_gemm_wide(int qtype, int mode, int mi, const GemmParams& p, hipStream_t s) {
  const bool routed = mode == kGrouped || mode == kGroupedGU || mode == kGroupedDown;
  if (routed && p.t % 8 != 0) return hipErrorInvalidValue;  // table length
  if (mode == kGrouped || mode == kGroupedDown)
    for (int i = 0; i < p.seg.nseg; ++i)
      if (p.seg.n[i] % 256 != 0) return hipErrorInvalidValue;  // routed tiles are whole column tiles
  if (mode == kGroupedGU) {
    // p.n: h columns (a multiple of 128), 128 per column tile
    if (mi != 8 || p.n % 128 != 0) return hipErrorInvalidValue;
    const uint32_t gcols = (uint32_t)(p.n / 128);
    if (qtype == kQ4_K) launch_wide_t<kQ4_K, kGroupedGU, 8>(p, gcols, s);
    else if (qtype == kQ5_K) launch_wide_t<kQ5_K, kGroupedGU, 8>(p, gcols, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (mode != kPlainF16 && mode != kMulti && mode != kGrouped && mode != kGroupedDown) return hipErrorInvalidValue;
  if ((mode == kGrouped || mode == kGroupedDown) && mi != 8) return hipErrorInvalidValue;
  const uint32_t cols = mode != kPlainF16 ? (uint32_t)p.seg.tile0[p.seg.nseg] : (uint32_t)((p.n + 255) / 256);
#define QP_WIDE_T(QT)                                                                              \
  if (mode == kGrouped) {                                                                          \
    launch_wide_t<QT, kGrouped, 8>(p, cols, s);                                                    \
  } else if (mode == kGroupedDown) {                                                               \
    launch_wide_t<QT, kGroupedDown, 8>(p, cols, s);                                                \
  } else if (mode == kMulti) {                                                                     \
    if (mi == 8) launch_wide_t<QT, kMulti, 8>(p, cols, s); else launch_wide_t<QT, kMulti, 4>(p, cols, s); \
  } else {                                                                                         \
    if (mi == 8) launch_wide_t<QT, kPlainF16, 8>(p, cols, s); else launch_wide_t<QT, kPlainF16, 4>(p, cols, s); \
  }
  switch (qtype) {
    case kQ6_K: QP_WIDE_T(kQ6_K) break;
    case kQ2_K: QP_WIDE_T(kQ2_K) break;
    case kQ4_K: QP_WIDE_T(kQ4_K) break;
    case kQ5_K: QP_WIDE_T(kQ5_K) break;
    default: return hipErrorInvalidValue;
  }
#undef QP_WIDE_T
  return hipGetLastError();
}

// K slices: tiles of 32 mi tokens x 256 / ks features, (mi, ks) = (2, 2),
// (2, 4) or (4, 2); k % (256 ks) == 0; plain mode.
hipError_t launch_gemm_wide_ks(int qtype, int mi, int ks, const GemmParams& p, hipStream_t s) {
  if (!((mi == 2 && (ks == 2 || ks == 4)) || (mi == 4 && ks == 2))) return hipErrorInvalidValue;
  const int bn = 256 / ks, bm = 32 * mi;
  const dim3 grid((uint32_t)((p.n + bn - 1) / bn), (uint32_t)((p.t + bm - 1) / bm));
#define QP_WIDE_KS(QT)                                                                                     \
  if (mi == 4)                                                                                             \
    hipLaunchKernelGGL((gemm_wide_kernel<QT, kPlainF16, 4, 2>), grid, dim3(NTW), 0, s, p);                 \
  else if (ks == 2)                                                                                        \
    hipLaunchKernelGGL((gemm_wide_kernel<QT, kPlainF16, 2, 2>), grid, dim3(NTW), 0, s, p);                 \
  else                                                                                                     \
    hipLaunchKernelGGL((gemm_wide_kernel<QT, kPlainF16, 2, 4>), grid, dim3(NTW), 0, s, p);
  switch (qtype) {
    case kQ6_K: QP_WIDE_KS(kQ6_K) break;
    case kQ2_K: QP_WIDE_KS(kQ2_K) break;
    case kQ4_K: QP_WIDE_KS(kQ4_K) break;
    case kQ5_K: QP_WIDE_KS(kQ5_K) break;
    default: return hipErrorInvalidValue;
  }
#undef QP_WIDE_KS
  return hipGetLastError();
}

}  // namespace qp
