// gemm_common.h -- definitions shared by the projection kernels: tile
// constants, launch parameters, and the epilogues that turn the f32
// accumulators into outputs (plain store, per-head RMSNorm, SiLU(gate)*up,
// route-weighted expert output).
//
// MFMA 32x32x16 result layout: register a of lane l holds
// D[8*(a/4) + 4*(l/32) + a%4][l%32] of a 32 x 32 tile.
#pragma once

#include "qp_device.h"
#include "qp_internal.h"

namespace qp {

constexpr int BM = kTileM, BN = kTileN, BK = 64, NT = 256, LDK = BK + 8;

enum Mode { kPlainF16 = 0, kPlainF32 = 1, kQkNorm = 2, kGateUp = 3, kDown = 4, kMulti = 5, kGrouped = 6, kGroupedGU = 7,
           kGroupedDown = 8 };

// Projections sharing one X fused into one launch of the tall kernel (mode
// kMulti): segment s owns the output-column tiles [tile0[s], tile0[s + 1]),
// with its own weights, output and epilogue.  A segment may reduce over one
// part of K only: its weights and activations start xoff weights into each
// row and it sums k of them (the halves of a split projection, each writing
// its partial sums to an output of its own).
constexpr int kMaxSeg = 5;
struct GemmSegments {
  int nseg;
  int tile0[kMaxSeg + 1];
  const uint8_t* w[kMaxSeg];  // first weight block of the segment's K part, row 0
  int n[kMaxSeg];
  int k[kMaxSeg];
  int64_t xoff[kMaxSeg];      // offset of the K part into each activation row (elements)
  float* y[kMaxSeg];
  int64_t ldy[kMaxSeg];
  const float* gain[kMaxSeg];
  int64_t gstride[kMaxSeg];
  int norm[kMaxSeg];  // 1: per-head RMSNorm epilogue, 0: plain
};

struct GemmParams {
  const uint8_t* w;      // W (or the gate tensors of all experts)
  const uint8_t* w2;     // up tensors of all experts (gate/up pass)
  int64_t rb;            // bytes per W row
  int64_t estride;       // bytes per expert tensor
  int n;                 // W rows (output features)
  int k;                 // reduction length (multiple of 256)
  const void* x;         // activations (f16 or f32), or the f32 h rows (down pass)
  int64_t ldx;
  int t;                 // tokens (plain / qknorm)
  float* y;
  int64_t ldy;
  const float* gain;
  int64_t gstride;
  int hd;
  float eps;
  // routed experts
  const int* tiles;      // 128-row kernel: [max_tiles][2] = expert, first row of its list; 256-row kernel:
                         // [max_tiles2][4] = expert, first row, rows, first compact row (0 rows past the tiles)
  const int* ntiles;     // 128-row kernel: tiles in the table
  const int* offsets;    // first compact row of each expert
  const int* counts;     // rows of each expert
  const int* list;       // compact row -> pair index (token * top_k + slot)
  int top_k;
  uint32_t* rowmax;      // per compact row: bits of max |h|
  float* hbuf;           // [pairs][inter]
  float* dbuf;           // [pairs][hidden]
  const float* weights;  // [pairs]
  GemmSegments seg;      // fused projections (kMulti)
  int64_t part_stride;   // 128-tile plain modes split over gridDim.z K parts: floats between partial outputs
  int vec_store;         // 128-tile kernel: output rows are 16-byte multiples (16-byte stores)
  // routed experts on the 256 x 256-tile kernel: a tile table of 256-row
  // tiles of the per-expert lists.  kGrouped (gate / up segments) and
  // kGroupedGU: X rows are the tokens list[row] / top_k; kGroupedGU stages
  // 128 gate rows (w) and the same 128 up rows (w2) of an expert and writes
  // SiLU(g) u as f32 rows of n columns.  kGroupedDown: X rows are the compact
  // rows themselves, output row r goes to pair list[r].
  int tcols;  // routed modes: column tiles (set by the launcher)
};

// Power of two bringing a row's largest |h| into [2^14, 2^15): binary16 then
// holds every value of the row without overflow (inverse: its reciprocal).
__device__ __forceinline__ float row_scale_from_max(uint32_t maxbits, bool inverse) {
  if (maxbits == 0) return 1.f;
  int be = (int)(maxbits >> 23);
  int sh = 141 - be;
  sh = sh < -100 ? -100 : (sh > 100 ? 100 : sh);
  return __builtin_ldexpf(1.f, inverse ? -sh : sh);
}

// Epilogue of a tile whose waves form 2 x 2, each owning WM rows x 64
// columns (MI = WM / 32 MFMA tiles along M, 2 along N).  `base` is the first
// output row (token, or compact row of the routed passes), m_rows the valid
// rows, n0 the first output column.  `red` is LDS scratch of 2 * 2 * WM
// floats, free once the main loop's last barrier has passed.
// `active` false: a wave holding no tile (the producer waves of the
// specialised kernel) only takes part in the epilogue's barriers.
// f32 store of a wave's block of MI x JB MFMA tiles (32 x 32 each) with
// 16-byte stores: each tile goes through a per-wave LDS buffer of 32 rows x
// 40 floats, written in the register layout and read back as rows of
// float4.  (One 4-byte store per value made the store instructions, not HBM,
// bound the epilogue.)  The pitch of 40 floats puts the two half-waves of a
// register write in different halves of the 64 banks.  The LDS operations of
// a wave complete in order, so the read-back sees the writes.
// Tile (i, j) covers the block's rows 32 i .. + 31 and columns col0 + 32 j ..
// + 31; rows >= m_rows and columns >= ncols are not written.  row_ptr(r)
// gives the start of the block's row r in memory (16-byte aligned rows).
template <int MI, int JB, typename RowPtr>
__device__ __forceinline__ void store_tiles_vec(float16v (&v)[MI][JB], int m_rows, int col0, int ncols, int lane,
                                                float* scr, RowPtr&& row_ptr) {
  constexpr int PITCH = 40;
  const int ln = lane;  // from the lane counter (see gemm_epilogue)
  const int l8 = ln >> 3;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) {
#pragma unroll
      for (int a = 0; a < 16; ++a)
        scr[(8 * (a >> 2) + 4 * (ln >> 5) + (a & 3)) * PITCH + (ln & 31)] = v[i][j][a];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((q & 1) == 0) asm volatile("" ::: "memory");  // two float4 in flight: the registers are nearly all taken
        const int rr = 8 * q + l8, cg = ln & 7;
        const float4v x = *(const float4v*)(scr + rr * PITCH + 4 * cg);
        const int row = 32 * i + rr;
        const int col = col0 + 32 * j + 4 * cg;
        float* const dst = row_ptr(row) + col;  // (computed by every lane: row_ptr may use wave shuffles)
        if (row < m_rows) {
          if (col + 3 < ncols) {
            *(float4v*)dst = x;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < ncols) dst[e] = x[e];
          }
        }
      }
      asm volatile("" ::: "memory");
    }
}

// Plain store of a 2 x 2 tile's wave block (WM x 64) into p.y (ldy % 4 == 0).
template <int MI>
__device__ __forceinline__ void store_block_vec(const GemmParams& p, float16v (&acc)[MI][2], int base, int m_rows,
                                                int n0, int wm, int wn, int lane, float* scr) {
  constexpr int WM = 32 * MI;
  const int r0 = base + WM * wm;
  store_tiles_vec<MI, 2>(acc, m_rows - WM * wm, n0 + 64 * wn, p.n, lane, scr,
                         [&](int r) __attribute__((always_inline)) { return p.y + (int64_t)(r0 + r) * p.ldy; });
}

// vec_scratch (32 x 40 floats of per-wave LDS): every mode stores through
// store_tiles_vec, 16 bytes at a time (the caller guarantees 16-byte output
// rows: ldy % 4 == 0, and for the routed passes n % 4 == 0); null: one
// 4-byte store per value.
template <int MODE, int MI>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, float16v (&acc)[MI][2], int base, int m_rows,
                                              int n0, int wm, int wn, int lane, float* red, bool active = true,
                                              float* vec_scratch = nullptr, float* sum_scratch = nullptr) {
  constexpr int WM = 32 * MI;
  if (!active) {
    if constexpr (MODE == kQkNorm) {
      if (sum_scratch) __syncthreads();
      __syncthreads();
    }
    return;
  }
  // The lane index from the hardware lane counter: lane-derived values here
  // are then not shared with the main loop's address setup, which would keep
  // them live across the loop past the register budget.
  lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  auto row_of = [&](int i, int a) { return WM * wm + 32 * i + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3); };

  if constexpr (MODE == kPlainF16 || MODE == kPlainF32) {
    if (vec_scratch) {
      store_block_vec<MI>(p, acc, base, m_rows, n0, wm, wn, lane, vec_scratch);
      return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 64 * wn + 32 * j + (lane & 31);
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int r = row_of(i, a);
          if (r < m_rows && col < p.n) p.y[(int64_t)(base + r) * p.ldy + col] = acc[i][j][a];
        }
      }
  } else if constexpr (MODE == kQkNorm) {
    // Sum of squares of each row over the wave's 64 columns, reduced across
    // the 32 lanes that share a row, parked in LDS; after one barrier a head
    // of 64 columns reads its wave's sum, a head of 128 adds the two waves'.
    constexpr int TM = 2 * WM;
    // this lane's two gains, loaded first so that their latency passes
    // under the row sums
    float g[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + 64 * wn + 32 * j + (lane & 31);
      const int head = col / p.hd;
      g[j] = col < p.n ? p.gain[(int64_t)head * p.gstride + (col - head * p.hd)] : 0.f;
    }
    if (sum_scratch && MI % 2 == 0) {
      // Through LDS instead of 5 dependent lane shuffles per row: after one
      // barrier (other waves may still read their last chunk or have copies
      // in flight until then) each wave owns 64 rows x 36 floats of
      // sum_scratch.  Per 64 rows (two MFMA tiles along M) every lane writes
      // its squares row-major, then lane l adds up row l with 16-byte reads.
      // (The row pitch of 36 floats keeps those reads free of conflicts.)
      __syncthreads();
      constexpr int SP = 36;
#pragma unroll
      for (int h = 0; h < MI / 2; ++h) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int rl = 32 * ii + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3);
            const int i = 2 * h + ii;
            sum_scratch[rl * SP + (lane & 31)] = acc[i][0][a] * acc[i][0][a] + acc[i][1][a] * acc[i][1][a];
          }
        const float4v* rowp = (const float4v*)(sum_scratch + lane * SP);
        float4v t4 = rowp[0];
#pragma unroll
        for (int q = 1; q < 8; ++q) t4 += rowp[q];
        red[wn * TM + WM * wm + 64 * h + lane] = (t4[0] + t4[1]) + (t4[2] + t4[3]);
        asm volatile("" ::: "memory");  // the next 64 rows overwrite the scratch
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          float v = acc[i][0][a] * acc[i][0][a] + acc[i][1][a] * acc[i][1][a];
#pragma unroll
          for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m, 64);
          if ((lane & 31) == 0) red[wn * TM + row_of(i, a)] = v;
        }
    }
    __syncthreads();
    const float inv_hd = 1.f / (float)p.hd;
    const bool pair_heads = p.hd == 128;
    if (vec_scratch) {
      // normalise in place, then the plain 16-byte store (same products in
      // the same order as below)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int r = row_of(i, a);
          const float ss = pair_heads ? red[r] + red[TM + r] : red[wn * TM + r];
          const float scale = __builtin_amdgcn_rsqf(ss * inv_hd + p.eps);  // v_rsq_f32 (about 1 ulp)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j][a] = acc[i][j][a] * scale * g[j];
        }
      store_block_vec<MI>(p, acc, base, m_rows, n0, wm, wn, lane, vec_scratch);
      return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int r = row_of(i, a);
        const float ss = pair_heads ? red[r] + red[TM + r] : red[wn * TM + r];
        const float scale = __builtin_amdgcn_rsqf(ss * inv_hd + p.eps);  // v_rsq_f32 (about 1 ulp)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + 64 * wn + 32 * j + (lane & 31);
          if (r < m_rows && col < p.n) p.y[(int64_t)(base + r) * p.ldy + col] = acc[i][j][a] * scale * g[j];
        }
      }
  } else if constexpr (MODE == kGateUp) {
    // acc[i][0] = gate, acc[i][1] = up for output column n0 + 32 wn + lane%32
    const int col = n0 + 32 * wn + (lane & 31);
    float16v hv[MI][1];
    // Row maxima of |h| over the wave's 32 columns: with sum_scratch (64 x 36
    // floats of this wave's own LDS, MI == 2) the values are written
    // row-major and lane l takes the maximum of row l with 16-byte reads;
    // otherwise 5 lane shuffles per row value.
    constexpr int SP = 36;
    const bool via_lds = sum_scratch != nullptr && MI == 2;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int r = row_of(i, a);
        const float g = acc[i][0][a], u = acc[i][1][a];
        const float h = g / (1.f + __expf(-g)) * u;
        hv[i][0][a] = h;
        const bool ok = r < m_rows && col < p.n;
        if (ok && !vec_scratch) p.hbuf[(int64_t)(base + r) * p.n + col] = h;
        float mx = ok ? __builtin_fabsf(h) : 0.f;
        if (via_lds) {
          sum_scratch[(32 * i + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3)) * SP + (lane & 31)] = mx;
        } else {
#pragma unroll
          for (int m = 1; m < 32; m <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, 64));
          if ((lane & 31) == 0 && r < m_rows) atomicMax(p.rowmax + base + r, __builtin_bit_cast(uint32_t, mx));
        }
      }
    if (via_lds) {
      const float4v* rowp = (const float4v*)(sum_scratch + lane * SP);
      float4v m4 = rowp[0];
#pragma unroll
      for (int q = 1; q < 8; ++q) {
        const float4v v4 = rowp[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) m4[e] = __builtin_fmaxf(m4[e], v4[e]);
      }
      const float mx = __builtin_fmaxf(__builtin_fmaxf(m4[0], m4[1]), __builtin_fmaxf(m4[2], m4[3]));
      const int r = WM * wm + lane;  // lane l holds row l of the wave's block
      if (r < m_rows) atomicMax(p.rowmax + base + r, __builtin_bit_cast(uint32_t, mx));
      asm volatile("" ::: "memory");
    }
    if (vec_scratch) {
      const int r0 = base + WM * wm;
      store_tiles_vec<MI, 1>(hv, m_rows - WM * wm, n0 + 32 * wn, p.n, lane, vec_scratch,
                             [&](int r) __attribute__((always_inline)) { return p.hbuf + (int64_t)(r0 + r) * p.n; });
    }
  } else {  // kDown
    if (vec_scratch) {
      // Lane l looks up row l of the wave's block (its pair and factor); the
      // accumulator rows take them by shuffle.  Scale in registers (same
      // products as below), then 16-byte rows into each pair's dbuf row.
      static_assert(WM <= 64, "one block row per lane");
      const int rl = min(WM * wm + (lane & (WM - 1)), m_rows - 1);
      const int pair_l = p.list[base + rl];
      const float f_l = row_scale_from_max(p.rowmax[base + rl], true) * p.weights[pair_l];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const float f = __shfl(f_l, 32 * i + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3), 64);
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j][a] = acc[i][j][a] * f;
        }
      store_tiles_vec<MI, 2>(acc, m_rows - WM * wm, n0 + 64 * wn, p.n, lane, vec_scratch,
                             [&](int r) __attribute__((always_inline)) {
                               return p.dbuf + (int64_t)__shfl(pair_l, r, 64) * p.n;
                             });
      return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int r = row_of(i, a);
        if (r >= m_rows) continue;
        const int pair = p.list[base + r];
        const float f = row_scale_from_max(p.rowmax[base + r], true) * p.weights[pair];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + 64 * wn + 32 * j + (lane & 31);
          if (col < p.n) p.dbuf[(int64_t)pair * p.n + col] = acc[i][j][a] * f;
        }
      }
  }
}

static inline int64_t row_bytes_of(int qtype, int64_t cols) {
  switch (qtype) {
    case kF16: return cols * 2;
    case kQ8_0: return (cols + 31) / 32 * 34;
    case kQ4_K: return (cols + 255) / 256 * 144;
    case kQ5_K: return (cols + 255) / 256 * 176;
    case kQ6_K: return (cols + 255) / 256 * 210;
    case kQ2_K: return (cols + 255) / 256 * 84;
    default: return -1;
  }
}

// The 256-token tile kernel (gemm_tall.hip) for the plain f16 and QK-norm modes.
hipError_t launch_gemm_tall(int qtype, int mode, dim3 grid, const GemmParams& p, hipStream_t s);

// The kernel with in-register weight decode (gemm_wide.hip): tiles of
// 32 * mi tokens x wide_cols() features, mi = 8 or 4; plain f16 or kMulti
// (segments of whole column tiles over one X).
bool wide_supported(int qtype, int mode);
int wide_cols();
hipError_t launch_gemm_wide(int qtype, int mode, int mi, const GemmParams& p, hipStream_t s);
// The projection kernel in ks K slices: tiles of 32 mi tokens x 256 / ks
// features, (mi, ks) = (2, 2), (2, 4) or (4, 2), k % (256 ks) == 0, K-quant
// weights, binary16 activations, plain mode.
hipError_t launch_gemm_wide_ks(int qtype, int mi, int ks, const GemmParams& p, hipStream_t s);

}  // namespace qp
