// gemm_tall.hip -- the 256-token tile of the dequant-on-load projection
//   Y[t, n] = sum_k X[t, k] * W[n, k]
// ("QK-norm models take the FP16 batched prefill", section "What changes":
// chunked batched prefill in FP16; the QK norm is per head).
//
// Why a separate kernel: the weight bytes of a 128-row tile are few
// (0.3-1 byte per weight) but each GGUF row lives in its own place in HBM.
// Loading them lane-per-row puts 32 rows into every load instruction, which
// keeps the vector address unit busy far longer than the MFMAs of a tile.
// Here the workgroup copies whole superblock columns of its 128 weight rows
// with contiguous loads (one row per wave instruction, one dword per lane)
// into an LDS staging area, one unit of K ahead, and decodes from LDS.  The
// 256-token height halves the decode work per flop compared with 128.
//
// Workgroup: 512 threads = 8 waves.  Four consumer waves (2 x 2, each 128
// tokens x 64 features, 4 x 2 MFMA tiles of 32 x 32, v_mfma_f32_32x32x16_f16
// with f32 accumulation) only read fragments and multiply; four producer waves
// only stage weight bytes and decode them.  Each SIMD runs one wave of each
// role, so decode arithmetic issues beside the MFMAs.  K advances in chunks of
// 64; per chunk:
//   * activations 256 x 64 (binary16) go straight from global memory into an
//     LDS ring (16-byte direct loads issued by the consumer waves one or two
//     chunks ahead, as deep as the LDS left over by the staging area allows);
//   * each producer thread decodes one 32-weight unit of one weight row from
//     the LDS staging copy into the binary16 weight tile (nearest-even of the
//     exact f32 value);
//   * 32 MFMAs per consumer wave.
// The staging area holds two units: while one is decoded, the producers fill
// the other with direct global-to-LDS dword loads issued over the first two
// chunks of the unit, and wait for them only at the barrier before the unit
// is needed, so no chunk pays for a whole unit's load latency.
// LDS tiles keep rows of 64 halfs (128 B) as 8 pieces of 16 B; piece p of row
// r sits in slot p ^ ((r >> 1) & 7).  The LDS serves a 16-byte read for 16
// lanes per cycle from 64 banks (256 B), i.e. two 128-byte rows: with this
// slot order the 16 consecutive rows of a fragment read fall in 16 different
// 16-byte bank groups (a plain p ^ (r & 7) would put rows r and r + 8 in the
// same group and halve the read rate).  The staging copy keeps RSD dwords per
// row with RSD odd, so dword reads of the 32 rows of a wave at one offset hit
// distinct banks.
#include <type_traits>

#include "gemm_common.h"

namespace qp {

constexpr int TBM = 256;           // tokens per tile
constexpr int TMI = TBM / 2 / 32;  // MFMA tiles per wave along M

// Staging unit of K per type: weights (KW), bytes per row (UB), LDS dwords
// per row (RSD >= (UB + 2 + 3) / 4, odd).
template <int QT> struct StageUnit;
template <> struct StageUnit<kQ4_K> { static constexpr int KW = 256, UB = 144, RSD = 37; };
template <> struct StageUnit<kQ5_K> { static constexpr int KW = 256, UB = 176, RSD = 45; };
template <> struct StageUnit<kQ6_K> { static constexpr int KW = 256, UB = 210, RSD = 53; };
template <> struct StageUnit<kQ2_K> { static constexpr int KW = 256, UB = 84, RSD = 21; };
template <> struct StageUnit<kQ8_0> { static constexpr int KW = 128, UB = 136, RSD = 35; };
// F16 weights are not staged: the producers copy each chunk's binary16 rows
// straight into the weight tile.  The small area only holds the epilogue's
// reduction scratch.
template <> struct StageUnit<kF16> { static constexpr int KW = 64, UB = 128, RSD = 5; };

constexpr int kLdsBytes = 160 * 1024;
// Weight tile ring: two buffers where the producers decode one chunk ahead;
// three for F16 weights, whose direct loads are issued two chunks ahead.
template <int QT>
constexpr int wbuf_of() {
  return QT == kF16 ? 3 : 2;
}
// Activation ring depth: three buffers where the LDS allows, else two.
template <int QT>
constexpr int xbuf_of() {
  return 3 * TBM * BK * 2 + wbuf_of<QT>() * BN * BK * 2 + 2 * BN * StageUnit<QT>::RSD * 4 <= kLdsBytes ? 3 : 2;
}
static_assert(BN * 5 >= 4 * TBM / 2 * 2 / 2, "staging area holds the epilogue reduction scratch");

template <int QT>
struct TallSmem {
  _Float16 x[xbuf_of<QT>()][TBM * BK];
  _Float16 w[wbuf_of<QT>()][BN * BK];
  uint32_t raw[2][BN * StageUnit<QT>::RSD];
};

// Workgroup barrier that waits for this wave's LDS reads and writes only.
// __syncthreads() also orders global memory, which makes the compiler drain
// every outstanding global load first, the direct-to-LDS copies included;
// the main loops keep those in flight across barriers and wait for them
// explicitly (s_waitcnt vmcnt) where their data is needed.
// The explicit wait is the builtin, so the compiler's own wait placement
// knows that every LDS read issued before the barrier has returned.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

// LDS offset (halfs) of 16-byte piece `piece` of tile row `row`
__device__ __forceinline__ int swz_of(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int piece) { return (row * 8 + (piece ^ swz_of(row))) * 8; }

// 8 dwords holding block bytes [f0, f0 + 32) of a staged row whose block
// starts `delta` (0 or 2) bytes into its first dword.
__device__ __forceinline__ void staged32(const uint32_t* row, uint32_t delta, uint32_t f0, uint32_t (&out)[8]) {
  const uint32_t b = delta + f0, k0 = b >> 2, s = b & 3;
  uint32_t d[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) d[i] = row[k0 + i];
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], s);
}

// the 16-bit field at block byte f (f even) of a staged row
__device__ __forceinline__ uint32_t staged16(const uint32_t* row, uint32_t delta, uint32_t f) {
  const uint32_t b = delta + f;
  return (row[b >> 2] >> (8 * (b & 3))) & 0xFFFFu;
}

// Decode 32-weight unit `ui` of a staged unit (a Q8_0 unit is 4 blocks; the
// K types' is one superblock) into the UnitRaw form of qp_device.h.
template <int QT> __device__ __forceinline__ void staged_unit(const uint32_t* row, uint32_t delta, uint32_t ui,
                                                             UnitRaw& r);

template <> __device__ __forceinline__ void staged_unit<kQ8_0>(const uint32_t* row, uint32_t delta, uint32_t ui,
                                                              UnitRaw& r) {
  const uint32_t f = 34 * ui;
  const float d = f16_to_f32(staged16(row, delta, f));
  staged32(row, delta, f + 2, r.code);
  r.a0 = r.a1 = d;
  r.b0 = r.b1 = 0.f;
  r.sm0 = r.sm1 = d;
}

template <> __device__ __forceinline__ void staged_unit<kQ4_K>(const uint32_t* row, uint32_t, uint32_t u, UnitRaw& r) {
  const uint32_t h0 = row[0], s0 = row[1], s1 = row[2], s2 = row[3];  // 144-byte blocks: delta is 0
  const float d = f16_to_f32(h0 & 0xFFFFu), dmin = f16_to_f32(h0 >> 16);
  uint32_t sc, m;
  q4k_scale_min(s0, s1, s2, u, sc, m);
  const uint32_t* qs = row + 4 + 8 * (u >> 1);
  const uint32_t sh = 4 * (u & 1);
#pragma unroll
  for (int j = 0; j < 8; ++j) r.code[j] = (qs[j] >> sh) & 0x0F0F0F0Fu;
  const float dsc = __fmul_rn(d, (float)sc);
  const float dm = __fmul_rn(dmin, (float)m);
  r.a0 = r.a1 = dsc;
  r.b0 = r.b1 = dm;
  r.sm0 = r.sm1 = dm;
}

template <> __device__ __forceinline__ void staged_unit<kQ5_K>(const uint32_t* row, uint32_t, uint32_t u, UnitRaw& r) {
  const uint32_t h0 = row[0], s0 = row[1], s1 = row[2], s2 = row[3];  // 176-byte blocks: delta is 0
  const float d = f16_to_f32(h0 & 0xFFFFu), dmin = f16_to_f32(h0 >> 16);
  uint32_t sc, m;
  q4k_scale_min(s0, s1, s2, u, sc, m);
  const uint32_t* qh = row + 4;
  const uint32_t* qs = row + 12 + 8 * (u >> 1);
  const uint32_t sh = 4 * (u & 1);
#pragma unroll
  for (int j = 0; j < 8; ++j) r.code[j] = ((qs[j] >> sh) & 0x0F0F0F0Fu) | (((qh[j] >> u) & 0x01010101u) << 4);
  const float dsc = __fmul_rn(d, (float)sc);
  const float dm = __fmul_rn(dmin, (float)m);
  r.a0 = r.a1 = dsc;
  r.b0 = r.b1 = dm;
  r.sm0 = r.sm1 = dm;
}

template <> __device__ __forceinline__ void staged_unit<kQ6_K>(const uint32_t* row, uint32_t delta, uint32_t u,
                                                              UnitRaw& r) {
  const uint32_t h = u >> 2, q4 = u & 3;
  // all 20 dwords first, one LDS round trip (the scheduler otherwise waits
  // for each field before reading the next)
  const uint32_t bl = delta + 64 * h + 32 * (q4 & 1), bh = delta + 128 + 32 * h;
  const uint32_t bs = delta + 192 + 2 * u, bd = delta + 208;
  uint32_t dl[9], dh[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) dl[i] = row[(bl >> 2) + i];
#pragma unroll
  for (int i = 0; i < 9; ++i) dh[i] = row[(bh >> 2) + i];
  const uint32_t wsc = row[bs >> 2], wd = row[bd >> 2];
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t scp = (wsc >> (8 * (bs & 3))) & 0xFFFFu;
  const float d = f16_to_f32((wd >> (8 * (bd & 3))) & 0xFFFFu);
  // one funnel shift per dword both undoes the field's byte offset in its
  // first dword and brings the wanted nibble (ql) or 2-bit field (qh) of each
  // byte to bit 0 (shift amounts at most 16 + 6)
  const uint32_t sa = 8 * (bl & 3) + 4 * (q4 >> 1), sb = 8 * (bh & 3) + 2 * q4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = __builtin_amdgcn_alignbit(dl[j + 1], dl[j], sa);
    const uint32_t hi = __builtin_amdgcn_alignbit(dh[j + 1], dh[j], sb);
    r.code[j] = (lo & 0x0F0F0F0Fu) | ((hi & 0x03030303u) << 4);
  }
  const float a0 = __fmul_rn(d, (float)(int8_t)(scp & 0xFFu));
  const float a1 = __fmul_rn(d, (float)(int8_t)(scp >> 8));
  r.a0 = a0;
  r.a1 = a1;
  r.b0 = __fmul_rn(a0, 32.f);
  r.b1 = __fmul_rn(a1, 32.f);
  r.sm0 = a0;
  r.sm1 = a1;
}

template <> __device__ __forceinline__ void staged_unit<kQ2_K>(const uint32_t* row, uint32_t, uint32_t u, UnitRaw& r) {
  const uint32_t* qs = row + 4 + 8 * (u >> 2);  // 84-byte blocks: delta is 0
  const uint32_t sh = 2 * (u & 3);
#pragma unroll
  for (int k = 0; k < 8; ++k) r.code[k] = (qs[k] >> sh) & 0x03030303u;
  const uint32_t scp = (row[u >> 1] >> (16 * (u & 1))) & 0xFFFFu;
  const uint32_t dd = row[20];
  const float d = f16_to_f32(dd & 0xFFFFu), dmin = f16_to_f32(dd >> 16);
  const uint32_t s0 = scp & 0xFFu, s1 = scp >> 8;
  r.a0 = __fmul_rn(d, (float)(s0 & 15u));
  r.a1 = __fmul_rn(d, (float)(s1 & 15u));
  r.b0 = __fmul_rn(dmin, (float)(s0 >> 4));
  r.b1 = __fmul_rn(dmin, (float)(s1 >> 4));
  r.sm0 = r.b0;
  r.sm1 = r.b1;
}

// Q2_K to binary16 by table: a sub-block's 16 weights take only the values
// v_q = RNE16(fma(d*sc, q, -dmin*m)), q = 0..3 (the same single-rounding f32
// value as unit_to_f16), so the four values are computed once and each
// weight picks its own with a byte permute.  The selector of two weights is
// the bytes (2 q0, 2 q0 + 1, 2 q1, 2 q1 + 1), itself one permute of 2 q and
// 2 q + 1.
__device__ __forceinline__ void q2k_unit_to_f16_lut(const UnitRaw& r, uint32_t (&out)[16]) {
  uint32_t t01[2], t23[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float a = h ? r.a1 : r.a0, b = h ? r.b1 : r.b0;
    t01[h] = pack_f16x2(__builtin_fmaf(a, 0.f, -b), __builtin_fmaf(a, 1.f, -b));
    t23[h] = pack_f16x2(__builtin_fmaf(a, 2.f, -b), __builtin_fmaf(a, 3.f, -b));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int h = j >> 2;
    const uint32_t e = r.code[j] << 1, o = e | 0x01010101u;   // 2 q and 2 q + 1 per byte
    const uint32_t s01 = __builtin_amdgcn_perm(o, e, 0x05010400u);
    const uint32_t s23 = __builtin_amdgcn_perm(o, e, 0x07030602u);
    out[2 * j] = __builtin_amdgcn_perm(t23[h], t01[h], s01);
    out[2 * j + 1] = __builtin_amdgcn_perm(t23[h], t01[h], s23);
  }
}

template <int QT, int MODE>
__global__ __launch_bounds__(2 * NT) void gemm_tall_kernel(GemmParams pk) {
  using SU = StageUnit<QT>;
  constexpr int RSD = SU::RSD, CPU = SU::KW / BK;  // chunks per staging unit
  constexpr int XB = xbuf_of<QT>();
  constexpr int WB = wbuf_of<QT>();
  // staging of the next unit is issued over the first NPART chunks of a unit
  // (all but its last chunk, at most three), each part a slice of the 32 rows
  // of a producer wave
  constexpr int NPART = CPU >= 4 ? 3 : 1;
  static_assert(sizeof(TallSmem<QT>) <= kLdsBytes, "LDS budget");
  __shared__ __attribute__((aligned(16))) TallSmem<QT> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Roles: waves of even bit parity {0, 3, 5, 6} multiply, {1, 2, 4, 7}
  // produce.  Whether a SIMD takes waves {i, i + 4} or {2i, 2i + 1} of the
  // workgroup, each SIMD then runs one of each.
  const bool producer = (__builtin_popcount(wave) & 1) != 0;
  const int role_idx = wave >> 1;  // 0..3 within each role
  // kMulti: this tile's projection (uniform per workgroup)
  // kMulti: this tile's projection (uniform per workgroup).  Its grid is
  // (token tiles, column tiles), so a segment's workgroups are issued
  // together, in segment order (whole-K segments first).
  GemmParams p = pk;
  int tile_x = MODE == kMulti ? blockIdx.y : blockIdx.x;
  const int tile_m = MODE == kMulti ? blockIdx.x : blockIdx.y;
  bool norm = MODE == kQkNorm;
  if constexpr (MODE == kMulti) {
    int sg = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i) sg += (i < pk.seg.nseg && tile_x >= pk.seg.tile0[i]);
    tile_x -= pk.seg.tile0[sg];
    p.w = pk.seg.w[sg];
    p.n = pk.seg.n[sg];
    p.k = pk.seg.k[sg];
    p.x = (const _Float16*)pk.x + pk.seg.xoff[sg];
    p.y = pk.seg.y[sg];
    p.ldy = pk.seg.ldy[sg];
    p.gain = pk.seg.gain[sg];
    p.gstride = pk.seg.gstride[sg];
    norm = pk.seg.norm[sg] != 0;
  }
  const int n0 = tile_x * BN;
  const int m0 = tile_m * TBM;
  const int m_rows = min(TBM, p.t - m0);
  const int nch = p.k / BK;
  const int nunits = p.k / SU::KW;

  const int wm = role_idx >> 1, wn = role_idx & 1;
  // Epilogue of this tile; the producer waves only take its barriers.  Each
  // role calls it from its own branch, so the accumulators are not live in
  // the producer code (whose decode then has the registers to issue all of a
  // unit's LDS reads at once).
  auto epilogue = [&](float16v(&acc)[TMI][2], bool active) __attribute__((always_inline)) {
    // reduction scratch in the staging area: no asynchronous copy writes there
    float* red = (float*)sm.raw[0];
    // per-wave transpose buffers of the plain store in the weight tiles: no
    // direct load targets them, and after the last barrier only the unused
    // next-chunk fragment reads touch them
    float* vec = (float*)sm.w[0] + 32 * 40 * role_idx;
    // QK-norm row sums: 64 x 36 floats per consumer wave in the activation
    // ring, free once every wave has passed the epilogue's first barrier
    float* sums = (float*)sm.x + 64 * 36 * role_idx;
    static_assert(sizeof(sm.x) >= 4 * 64 * 36 * sizeof(float), "activation ring holds the row-sum scratch");
    if constexpr (MODE == kMulti) {
      if (norm)
        gemm_epilogue<kQkNorm, TMI>(p, acc, m0, m_rows, n0, wm, wn, lane, red, active, vec, sums);
      else
        gemm_epilogue<kPlainF16, TMI>(p, acc, m0, m_rows, n0, wm, wn, lane, red, active, vec);
    } else {
      gemm_epilogue<MODE, TMI>(p, acc, m0, m_rows, n0, wm, wn, lane, red, active, vec, sums);
    }
  };

  if (!producer) {
    // The consumer (the MFMA feeder) issues ahead of the producer on its
    // SIMD; by default the older wave of a pair wins, which made the two
    // halves of the tile finish a chunk at different times.
    __builtin_amdgcn_s_setprio(1);
    // ---- consumer waves -------------------------------------------------
    float16v acc[TMI][2];
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = (float16v){};
    // Activation copy: this wave's 8 load instructions cover tile rows
    // 64 cw + 8 q .. + 7; lane l lands in slot l & 7 of row 64 cw + 8 q + (l >> 3),
    // which holds the piece that slot order puts there.
    const int cw = role_idx;
    const _Float16* xtile = (const _Float16*)p.x + (int64_t)m0 * p.ldx;  // tile row 0
    uint32_t xoff[8];  // bytes from xtile (a tile spans under 2^31 bytes)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 64 * cw + 8 * q + (lane >> 3);
      const int piece = (lane & 7) ^ swz_of(row);
      xoff[q] = (uint32_t)(2 * (min(row, m_rows - 1) * p.ldx + 8 * piece));
    }
    // load q (of 8) of this wave's share of chunk c (past the end: the last
    // chunk again), as a buffer load over the tile's rows: the lane's byte
    // offset is fixed and the chunk's goes in the scalar offset, so a load
    // costs no vector address arithmetic.
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)xtile, (short)0, -1, 0x00020000);
    auto load_xq = [&](int c, int q) __attribute__((always_inline)) {
      c = c < nch ? c : nch - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc,
                                               (__attribute__((address_space(3))) void*)(sm.x[c % XB] + (64 * cw + 8 * q) * BK),
                                               16, (int)xoff[q], 128 * c, 0, 0);
    };
    // Chunk j goes to buffer j % XB and is loaded right after the barrier
    // that ends the reads of chunk j - XB (the prologue loads chunks
    // 0 .. XB - 1).  Waiting for chunk c + 1 at the end of chunk c leaves the
    // loads of chunks c + 2 .. c + XB - 1 in flight.
    auto wait_x = [&]() __attribute__((always_inline)) {
      if constexpr (XB == 3)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // Fragment reads of step s: rows 32 apart share the slot order (it
    // depends on row bits 1..3), so one address per step and buffer serves
    // all of them, the 32-row strides going into the reads' immediate offset.
    auto frags = [&](const _Float16* xs, const _Float16* ws, int s, half8 (&a)[TMI], half8 (&b)[2]) {
      const int piece = 2 * s + (lane >> 5);
      const _Float16* pa = xs + swz(128 * wm + (lane & 31), piece);
      const _Float16* pb = ws + swz(64 * wn + (lane & 31), piece);
#pragma unroll
      for (int i = 0; i < TMI; ++i) a[i] = *(const half8*)(pa + 32 * BK * i);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const half8*)(pb + 32 * BK * j);
    };
    auto mfmas = [&](const half8 (&a)[TMI], const half8 (&b)[2]) {
#pragma unroll
      for (int i = 0; i < TMI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    };
    // The same MFMAs, each followed by one activation load of chunk cl: a
    // load's issue can stall on a full address queue, which costs nothing
    // while the MFMA before it runs.  (The loads sit here in program order:
    // the compiler does not move direct-to-LDS loads past LDS reads.)
    auto mfmas_loading = [&](const half8 (&a)[TMI], const half8 (&b)[2], int cl) {
      static_assert(2 * TMI == 8, "one activation load per MFMA of a step");
#pragma unroll
      for (int i = 0; i < TMI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
          load_xq(cl, 2 * i + j);
        }
    };
#pragma unroll
    for (int c = 0; c < XB; ++c)
#pragma unroll
      for (int q = 0; q < 8; ++q) load_xq(c, q);
    lds_barrier();  // first unit staged
    if constexpr (XB == 3)  // chunk 0 landed
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    lds_barrier();  // first chunk decoded
    constexpr int NF = TMI + 2, NM = 2 * TMI;
    // Rotated loop: the barrier that hands over chunk c + 1 sits after the
    // last fragment reads of chunk c, and the reads of chunk c + 1's steps 0
    // and 1 go out right after it, between the MFMAs of chunk c's steps 2 and
    // 3, so the matrix unit does not wait for LDS at the start of a chunk.
    // Buffers stay safe: the next writes to chunk c's X and W slots are issued
    // after that barrier, which every wave passes only once all of its reads
    // of chunk c have returned.  (After the last chunk the reads fetch unused
    // values from in-bounds LDS.)
    half8 a0[TMI], b0[2], a1[TMI], b1[2];  // steps 0 and 1 of the current chunk
    frags(sm.x[0], sm.w[0], 0, a0, b0);
    frags(sm.x[0], sm.w[0], 1, a1, b1);
    for (int c = 0; c < nch; ++c) {
      const _Float16* xs = sm.x[c % XB];
      const _Float16* ws = sm.w[c % WB];
      half8 a2[TMI], b2[2], a3[TMI], b3[2];
      mfmas(a0, b0);
      frags(xs, ws, 2, a2, b2);
      mfmas(a1, b1);
      frags(xs, ws, 3, a3, b3);
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // step 0 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);  // step 2 reads
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // step 1 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);  // step 3 reads
      __builtin_amdgcn_sched_barrier(0);
      wait_x();         // chunk c + 1 landed
      lds_barrier();    // chunk c + 1 decoded; this wave's reads of chunk c are done
      __builtin_amdgcn_sched_barrier(0);
      const _Float16* xn = sm.x[(c + 1) % XB];
      const _Float16* wnx = sm.w[(c + 1) % WB];
      frags(xn, wnx, 0, a0, b0);
      mfmas_loading(a2, b2, c + XB);  // chunk c's buffer is free: load chunk c + XB
      frags(xn, wnx, 1, a1, b1);
      mfmas(a3, b3);
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);  // next chunk's step 0 reads
#pragma unroll
      for (int i = 0; i < NM; ++i) {                        // step 2 MFMAs, each followed by
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an activation load
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);  // next chunk's step 1 reads
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // step 3 MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped re-loads past the end have landed
    epilogue(acc, true);
  } else if constexpr (QT == kF16) {
    // ---- producer waves, F16 weights: copy rows into the weight tile ------
    // Wave pw fills tile rows 32 pw .. + 31 of each chunk with 4 direct
    // 16-byte loads per lane, laid out like the activation copy (lane l lands
    // in slot l & 7 of row 32 pw + 8 q + (l >> 3), which holds the piece the
    // slot order puts there).  Rows past the tensor repeat its last row.
    // Chunk c + 2 is issued into its ring slot right after the barrier that
    // ends the reads of chunk c - 1, the slot's previous chunk, and waited
    // for at the barrier that hands over chunk c + 1.
    const int pw = role_idx;
    const __amdgpu_buffer_rsrc_t wrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.w + (int64_t)n0 * p.rb), (short)0, -1, 0x00020000);
    uint32_t woff[4];  // bytes from row n0 (128 rows span under 2^31 bytes)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 32 * pw + 8 * q + (lane >> 3);
      const int piece = (lane & 7) ^ swz_of(row);
      woff[q] = (uint32_t)(min(row, p.n - 1 - n0) * p.rb + 16 * piece);
    }
    auto load_w = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc,
                                                 (__attribute__((address_space(3))) void*)(sm.w[c % WB] + (32 * pw + 8 * q) * BK),
                                                 16, (int)woff[q], 128 * c, 0, 0);
    };
    load_w(0);
    load_w(1);  // K is a multiple of 256: at least 4 chunks
    lds_barrier();
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // chunk 0 landed
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
      if (c + 2 < nch) {
        load_w(c + 2);
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // chunk c + 1 landed
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();  // chunk c + 1 in place; the consumers' reads of chunk c are done
    }
    float16v none[TMI][2];  // not read: the producer side of the epilogue only synchronises
    epilogue(none, false);
  } else {
    // ---- producer waves: stage and decode ---------------------------------
    const int pw = role_idx;  // 0..3
    // Staging: rows pw + 4 r, r in [R0, R1), of unit u; one direct load per
    // row puts dword `lane` of the row's unit bytes (from the dword holding its
    // first byte) at dword `lane` of the row's slot.  Lanes past the unit's
    // last dword load nothing.
    // A full tile (every row inside the tensor) stages from one wave-uniform
    // address stepping 4 rows: rows 4 apart start at the same offset within a
    // dword (4 row strides are a multiple of 4 bytes), so the lanes and the
    // dword count are the same for all of them and the per-row cost is a few
    // scalar adds (the scalar unit is shared by the CU's four SIMDs).
    const bool full_tile = n0 + BN <= p.n;
    auto stage_rows = [&](int u, auto r0c, auto r1c) __attribute__((always_inline)) {
      constexpr int R0 = decltype(r0c)::value, R1 = decltype(r1c)::value;
      uint32_t* dst = sm.raw[u & 1];
      const int64_t uoff = (int64_t)u * SU::UB;
      const int64_t step = 4 * p.rb;
      if (full_tile) {
        const uint8_t* first = p.w + (int64_t)(n0 + pw + 4 * R0) * p.rb + uoff;
        const uint32_t a = (uint32_t)((uintptr_t)first & 3);
        const uint32_t cnt = (a + SU::UB + 3) >> 2;
        const uint8_t* base = first - a;
        if ((uint32_t)lane < cnt) {
#pragma unroll
          for (int r = R0; r < R1; ++r, base += step)
            __builtin_amdgcn_global_load_lds((const void*)((const uint32_t*)base + lane),
                                             (__attribute__((address_space(3))) void*)(dst + (pw + 4 * r) * RSD), 4,
                                             0, 0);
        }
        return;
      }
      const uint8_t* last = p.w + (int64_t)(p.n - 1) * p.rb + uoff;  // rows past the tensor repeat its last row
      const uint8_t* rp = p.w + (int64_t)(n0 + pw + 4 * R0) * p.rb + uoff;
#pragma unroll
      for (int r = R0; r < R1; ++r, rp += step) {
        const int n = pw + 4 * r;
        const uint8_t* blk = n0 + n < p.n ? rp : last;
        const uint32_t cnt = (uint32_t)((((uintptr_t)blk & 3) + SU::UB + 3) >> 2);
        if ((uint32_t)lane < cnt)
          __builtin_amdgcn_global_load_lds((const void*)(dword_floor(blk) + lane),
                                           (__attribute__((address_space(3))) void*)(dst + n * RSD), 4, 0, 0);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, BN / 4 * 1 / NPART>;
    using I2 = std::integral_constant<int, BN / 4 * 2 / NPART>;
    using IE = std::integral_constant<int, BN / 4>;
    // decode: producer thread owns weight row pt & 127 of the tile, 32-weight
    // half kh = pt >> 7, so the 64 lanes of a wave read 64 different staged
    // rows at one offset, which an odd row pitch spreads over all 64 banks
    // (two lanes per row would read 8 dwords apart, and some row pairs collide).
    const int pt = pw * 64 + lane;  // 0..255
    const int wn_t = pt & 127, kh = pt >> 7;
    const uint8_t* wrow = p.w + (int64_t)min(n0 + wn_t, p.n - 1) * p.rb;
    auto decode = [&](int c, int buf) __attribute__((always_inline)) {
      const int u = c / CPU;
      const uint32_t delta = (uint32_t)(((uintptr_t)wrow + (uintptr_t)u * SU::UB) & 3);
      UnitRaw ur;
      staged_unit<QT>(sm.raw[u & 1] + wn_t * RSD, delta, (uint32_t)(2 * (c % CPU) + kh), ur);
      uint32_t hw[16];
      if constexpr (QT == kQ2_K)
        q2k_unit_to_f16_lut(ur, hw);
      else
        unit_to_f16<QT>(ur, hw);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(u32x4*)(sm.w[buf] + swz(wn_t, 4 * kh + q)) = (u32x4){hw[4 * q], hw[4 * q + 1], hw[4 * q + 2], hw[4 * q + 3]};
    };
    // Unit u + 1 is staged while chunks of unit u are decoded: part ph after
    // the decode of the unit's chunk ph (ph < NPART; by then the activation
    // loads issued at the start of the chunk are mostly served), complete at
    // its last chunk.  Its buffer last held unit u - 1, whose final decode
    // preceded the previous barrier.
    auto stage_next = [&](int c) __attribute__((always_inline)) {
      const int u = c / CPU, ph = c % CPU;
      if (u + 1 >= nunits) return;
      if constexpr (NPART == 1) {
        if (ph == 0) stage_rows(u + 1, I0{}, IE{});
      } else {
        static_assert(NPART == 3, "three staging parts");
        if (ph == 0)
          stage_rows(u + 1, I0{}, I1{});
        else if (ph == 1)
          stage_rows(u + 1, I1{}, I2{});
        else if (ph == 2)
          stage_rows(u + 1, I2{}, IE{});
      }
    };

    stage_rows(0, I0{}, IE{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // first unit staged
    decode(0, 0);
    stage_next(0);
    lds_barrier();  // first chunk decoded
    for (int c = 0; c < nch; ++c) {
      const int nc = c + 1;
      if (nc < nch) {
        decode(nc, nc & 1);
        stage_next(nc);
        if (nc % CPU == CPU - 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // next unit staged
      }
      lds_barrier();  // next chunk decoded
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float16v none[TMI][2];  // not read: the producer side of the epilogue only synchronises
    epilogue(none, false);
  }
}

hipError_t launch_gemm_tall(int qtype, int mode, dim3 grid, const GemmParams& p, hipStream_t s) {
#define QP_TALL(QT)                                                                          \
  if (mode == kQkNorm)                                                                       \
    hipLaunchKernelGGL((gemm_tall_kernel<QT, kQkNorm>), grid, dim3(2 * NT), 0, s, p);        \
  else if (mode == kMulti)                                                                   \
    hipLaunchKernelGGL((gemm_tall_kernel<QT, kMulti>), grid, dim3(2 * NT), 0, s, p);         \
  else                                                                                       \
    hipLaunchKernelGGL((gemm_tall_kernel<QT, kPlainF16>), grid, dim3(2 * NT), 0, s, p);
  switch (qtype) {
    case kF16: QP_TALL(kF16) break;
    case kQ8_0: QP_TALL(kQ8_0) break;
    case kQ4_K: QP_TALL(kQ4_K) break;
    case kQ5_K: QP_TALL(kQ5_K) break;
    case kQ6_K: QP_TALL(kQ6_K) break;
    case kQ2_K: QP_TALL(kQ2_K) break;
    default: return hipErrorInvalidValue;
  }
#undef QP_TALL
  return hipGetLastError();
}

}  // namespace qp
