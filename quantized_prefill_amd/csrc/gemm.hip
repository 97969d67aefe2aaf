// gemm.hip -- dequant-on-load FP16 MFMA projection for gfx950, its per-head
// RMSNorm epilogue, and the two passes of the routed grouped-expert FFN.
//
//   Y[t, n] = sum_k X[t, k] * W[n, k]
// ("QK-norm models take the FP16 batched prefill", section "What changes":
// a chunk of prompt tokens runs through each projection as one FP16
// product; the QK norm is per head.)
//
// This file holds the 128-token tile kernel (small token counts, the routed
// expert passes, f32 activations), the router and the routed-expert list
// kernels; gemm_tall.hip holds the 256-token tile kernel used for large
// prefill chunks.
//
// Tiling here: a workgroup of 256 threads (4 waves of 64) owns a 128 (tokens)
// x 128 (output features) tile of Y and walks K in chunks of 64.  Per chunk:
//   * X: 128 x 64 activations -> LDS as binary16 (f32 inputs are rounded to
//     nearest-even on the way).
//   * W: each thread decodes one 32-weight unit of one W row straight from the
//     GGUF blocks in HBM (nearest-even binary16 of the exact f32 value) into
//     LDS.  W is never materialised in HBM.
//   * each wave multiplies its 64 x 64 sub-tile with v_mfma_f32_32x32x16_f16
//     (2 x 2 tiles of 32 x 32, f32 accumulators), 4 k-steps of 16.
// LDS is double-buffered: the global loads of chunk c+1 are issued before the
// MFMAs of chunk c and decoded into the other buffer after them, with one
// barrier per chunk.  LDS rows are padded to 72 halfs (144 B), which keeps the
// 16-byte fragment reads of 32 consecutive rows free of bank conflicts.
//
// MFMA 32x32x16 operand layout (lane l, 8 halfs per lane): A row l%32 (B
// column l%32), k = 8*(l/32) + e; result register a of lane l holds
// D[8*(a/4) + 4*(l/32) + a%4][l%32].
#include <algorithm>
#include <type_traits>
#include <mutex>
#include <vector>

#include "gemm_common.h"

namespace qp {

struct GemmSmem {
  _Float16 x[2][BM * LDK];
  _Float16 w[2][BN * LDK];
};

template <int QT, int MODE>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmParams p) {
  using F = Fmt<QT>;
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile coordinates -------------------------------------------------
  int m_rows;        // valid rows of this tile
  int base = 0;      // first compact row (routed passes)
  int e = 0;         // expert
  int n0;            // first output column
  if constexpr (MODE == kGateUp || MODE == kDown) {
    const int tile = blockIdx.x;
    if (tile >= *p.ntiles) return;
    e = p.tiles[2 * tile];
    const int mstart = p.tiles[2 * tile + 1];
    base = p.offsets[e] + mstart;
    m_rows = min(BM, p.counts[e] - mstart);
    n0 = blockIdx.y * (MODE == kGateUp ? BN / 2 : BN);
  } else {
    n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    m_rows = min(BM, p.t - m0);
    base = m0;
    // K split over gridDim.z parts of p.k weights each: part z starts
    // z * p.k weights into every W and X row and writes its partial sums to
    // its own dense output
    if (gridDim.z > 1) {
      const int z = blockIdx.z;
      p.w += (int64_t)z * (p.k / F::QK) * F::TS;
      p.x = (const char*)p.x + (int64_t)z * p.k * (MODE == kPlainF32 ? 4 : 2);
      p.y += (int64_t)z * p.part_stride;
    }
  }

  // ---- per-thread activation rows ---------------------------------------
  // f16 rows: thread loads rows (tid >> 3) + 32 i, 16 bytes at column 8*(tid & 7)
  // f32 rows: thread loads rows (tid >> 4) + 16 i, 16 bytes at column 4*(tid & 15)
  constexpr bool XF32 = (MODE == kPlainF32 || MODE == kDown);
  constexpr int XR = XF32 ? 8 : 4;
  const char* xrow[XR];
  float xscale[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    int r = XF32 ? (tid >> 4) + 16 * i : (tid >> 3) + 32 * i;
    r = min(r, m_rows - 1);
    xscale[i] = 1.f;
    if constexpr (MODE == kGateUp) {
      const int tok = p.list[base + r] / p.top_k;
      xrow[i] = (const char*)((const _Float16*)p.x + (int64_t)tok * p.ldx);
    } else if constexpr (MODE == kDown) {
      xrow[i] = (const char*)(p.hbuf + (int64_t)(base + r) * p.k);
      xscale[i] = row_scale_from_max(p.rowmax[base + r], false);
    } else if constexpr (XF32) {
      xrow[i] = (const char*)((const float*)p.x + (int64_t)(base + r) * p.ldx);
    } else {
      xrow[i] = (const char*)((const _Float16*)p.x + (int64_t)(base + r) * p.ldx);
    }
  }
  const int xcol = XF32 ? 4 * (tid & 15) : 8 * (tid & 7);

  // ---- per-thread W row ---------------------------------------------------
  const int wn_t = tid >> 1, kh = tid & 1;
  const uint8_t* wrow;
  {
    if constexpr (MODE == kGateUp) {
      const int which = (wn_t >> 5) & 1;  // 0: gate, 1: up
      int gr = n0 + 32 * (wn_t >> 6) + (wn_t & 31);
      gr = min(gr, p.n - 1);
      wrow = (which ? p.w2 : p.w) + (int64_t)e * p.estride + (int64_t)gr * p.rb;
    } else {
      int gr = min(n0 + wn_t, p.n - 1);
      wrow = p.w + (int64_t)e * p.estride + (int64_t)gr * p.rb;
    }
  }

  u32x4 xv[XF32 ? 8 : 4];
  Raw<QT> wr;

  auto issue_loads = [&](int c) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if constexpr (XF32)
        xv[i] = *(const u32x4*)((const float*)xrow[i] + 64 * c + xcol);
      else
        xv[i] = *(const u32x4*)((const _Float16*)xrow[i] + 64 * c + xcol);
    }
    const int ui = 2 * c + kh;  // 32-weight unit index within the row
    wr.load(wrow + (int64_t)(ui / F::UNITS) * F::TS, (uint32_t)(ui % F::UNITS));
  };

  auto store_lds = [&](int buf) {
    _Float16* xs = sm.x[buf];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if constexpr (XF32) {
        const int r = (tid >> 4) + 16 * i;
        float4v f = __builtin_bit_cast(float4v, xv[i]);
        const float s = xscale[i];
        const uint32_t lo = pack_f16x2(f.x * s, f.y * s), hi = pack_f16x2(f.z * s, f.w * s);
        *(uint2*)(xs + r * LDK + xcol) = make_uint2(lo, hi);
      } else {
        const int r = (tid >> 3) + 32 * i;
        *(u32x4*)(xs + r * LDK + xcol) = xv[i];
      }
    }
    uint32_t hw[16];
    if constexpr (QT == kF16) {
      wr.halves(hw);
    } else {
      UnitRaw ur;
      wr.finish(ur);
      unit_to_f16<QT>(ur, hw);
    }
    _Float16* ws = sm.w[buf] + wn_t * LDK + 32 * kh;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(u32x4*)(ws + 8 * q) = (u32x4){hw[4 * q], hw[4 * q + 1], hw[4 * q + 2], hw[4 * q + 3]};
  };

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (float16v){};

  const int nch = p.k / BK;
  issue_loads(0);
  store_lds(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) issue_loads(c + 1);
    const _Float16* xs = sm.x[buf];
    const _Float16* ws = sm.w[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 a[2], b[2];
      const int koff = 16 * s + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const half8*)(xs + (64 * wm + 32 * i + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const half8*)(ws + (64 * wn + 32 * j + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (c + 1 < nch) store_lds(buf ^ 1);
    __syncthreads();
  }

  // after the loop's last barrier the tiles are free: the norm's row sums
  // (2 x 2 x 64 floats), one 32 x 40 transpose buffer per wave, and 64 x 36
  // floats per wave for the row reductions (sums of squares, maxima of |h|)
  float* const lds = (float*)&sm;
  static_assert(sizeof(GemmSmem) >= (2 * 2 * 64 + 4 * 32 * 40 + 4 * 64 * 36) * 4, "epilogue scratch");
  gemm_epilogue<MODE, 2>(p, acc, base, m_rows, n0, wm, wn, lane, lds,
                         true, p.vec_store ? lds + 2 * 2 * 64 + 32 * 40 * wave : nullptr,
                         MODE == kGateUp || MODE == kQkNorm ? lds + 2 * 2 * 64 + 4 * 32 * 40 + 64 * 36 * wave
                                                            : nullptr);
}

template <int MODE>
static hipError_t launch_mode(int qtype, dim3 grid, const GemmParams& p, hipStream_t s) {
  switch (qtype) {
    case kF16: hipLaunchKernelGGL((gemm_kernel<kF16, MODE>), grid, dim3(NT), 0, s, p); break;
    case kQ8_0: hipLaunchKernelGGL((gemm_kernel<kQ8_0, MODE>), grid, dim3(NT), 0, s, p); break;
    case kQ4_K: hipLaunchKernelGGL((gemm_kernel<kQ4_K, MODE>), grid, dim3(NT), 0, s, p); break;
    case kQ5_K: hipLaunchKernelGGL((gemm_kernel<kQ5_K, MODE>), grid, dim3(NT), 0, s, p); break;
    case kQ6_K: hipLaunchKernelGGL((gemm_kernel<kQ6_K, MODE>), grid, dim3(NT), 0, s, p); break;
    case kQ2_K: hipLaunchKernelGGL((gemm_kernel<kQ2_K, MODE>), grid, dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Token-tile height: 256 halves the decode work per flop and is used when the
// launch still fills the 256 CUs with one 256-token tile each.  The tall
// kernel addresses a tile's activation rows with 32-bit byte offsets and
// stores outputs 16 bytes at a time (rows of Y a multiple of 16 bytes).
static bool tall_strides_ok(int64_t ldx, int64_t ldy) {
  return 256 * ldx * 2 < ((int64_t)1 << 31) && ldy % 4 == 0;
}
// F16 weight rows are copied with 32-bit byte offsets from a tile's first
// row: 128 rows must span under 2^31 bytes.
static bool tall_weights_ok(int qtype, int64_t k) {
  return qtype != kF16 || 128 * row_bytes_of(qtype, k) < ((int64_t)1 << 31);
}
static bool use_tall_tiles(int qtype, int64_t n, int64_t k, int64_t t, int64_t ldx, int64_t ldy) {
  const int64_t tiles = ((n + BN - 1) / BN) * ((t + 255) / 256);
  return t >= 512 && tiles >= 256 && tall_strides_ok(ldx, ldy) && tall_weights_ok(qtype, k);
}

// The kernel with weights decoded into registers (256 x 256 tiles) where its
// tiles fill the GPU in whole rounds (or at least two): its tiles do twice
// the work of the 256 x 128 tall tile, so a partly filled last round costs
// twice as much.
static bool wide_fills(int64_t tiles) {
  const int cus = cu_count();
  return tiles >= cus && (tiles % cus == 0 || tiles >= 2 * cus);
}
static bool use_wide_tiles(int qtype, int mode, int64_t n, int64_t t, int64_t ldx, int64_t ldy) {
  if (!wide_supported(qtype, mode) || !tall_strides_ok(ldx, ldy)) return false;
  const int64_t cols = (n + wide_cols() - 1) / wide_cols();
  return wide_fills(cols * ((t + 255) / 256));
}

// y[r, c] = y[r, c] + part[r, c] (part dense, row stride n): the second K
// half added to the first.  One thread per 4 columns of a row.
__global__ __launch_bounds__(256) void add_partial_kernel(const float* __restrict__ part, float* __restrict__ y,
                                                          int64_t ldy, int t, int n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (n + 3) / 4;
  if (i >= (int64_t)t * q) return;
  const int r = (int)(i / q), c = 4 * (int)(i - (int64_t)r * q);
  float* yr = y + (int64_t)r * ldy;
  const float* pr = part + (int64_t)r * n;
  if (c + 4 <= n && ldy % 4 == 0 && n % 4 == 0) {
    const float4v a = *(const float4v*)(yr + c), b = __builtin_nontemporal_load((const float4v*)(pr + c));  // part: read once
    *(float4v*)(yr + c) = a + b;
  } else {
    for (int e = c; e < n && e < c + 4; ++e) yr[e] = yr[e] + pr[e];
  }
}

// Sum of a plain projection's K parts, in part order:
// y[r, c] = (..((p_0 + p_1) + p_2) ..) + p_{S-1}, partials dense (row stride n)
// and part_stride floats apart.  One thread per 4 columns of a row.
__global__ __launch_bounds__(256) void ksplit_sum_kernel(const float* __restrict__ part, int64_t part_stride,
                                                         int nparts, float* __restrict__ y, int64_t ldy, int t,
                                                         int n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (n + 3) / 4;
  if (i >= (int64_t)t * q) return;
  const int64_t r = i / q;
  const int c = (int)(i - r * q) * 4;
  const float* src = part + r * n + c;
  float* dst = y + r * ldy + c;
  for (int e = 0; e < 4 && c + e < n; ++e) {
    float v = src[e];
    for (int z = 1; z < nparts; ++z) v = v + src[(int64_t)z * part_stride + e];
    dst[e] = v;
  }
}

// The 256 x 256-tile kernel in two K halves: for a launch of exactly half a
// round of those tiles (the 8B layer's down at T = 2048: 128 tiles), each
// half runs as one segment of one launch, a full round together; half 0
// writes y, half 1 dense partial sums, and one pass adds them in that order.
// The partial sums fill t * n floats, at most 128 tiles of 256 x 256 on a
// 256-CU GPU: 32 MiB.  (Taken for Q2_K weights and K >= 8192; see below.)
bool wide_halves_shape(int64_t n, int64_t k, int64_t t) {
  const int64_t tiles = ((n + 255) / 256) * ((t + 255) / 256);
  return k % 512 == 0 && k >= 8192 && 2 * tiles == cu_count();
}

// The projection kernel in K slices, for launches that the 256 x 256 tiles
// and the tall tiles leave short of the CUs: of the tilings 64 x 64 (four
// slices), 64 x 128 and 128 x 128 (two slices), the one with the most
// workgroups that still fit one round; none if none fits.
static bool wide_ks_choice(int64_t n, int64_t k, int64_t t, int& mi, int& ks) {
  const int64_t cus = cu_count();
  const int cand[3][2] = {{2, 4}, {2, 2}, {4, 2}};
  int64_t best = 0;
  for (const auto& c : cand) {
    const int64_t wgs = ((n + 256 / c[1] - 1) / (256 / c[1])) * ((t + 32 * c[0] - 1) / (32 * c[0]));
    if (k % (256 * c[1]) == 0 && wgs <= cus && wgs > best) {
      best = wgs;
      mi = c[0];
      ks = c[1];
    }
  }
  return best > 0;
}

// K parts for a plain 128-tile launch that leaves the GPU under-filled: the
// largest power of two (at most 8) whose parts still fit one round of
// workgroups (a second, partly filled round costs more than the split
// saves), with parts of whole 256-weight blocks.  1: no split.
int gemm_ksplit_parts(int64_t n, int64_t k, int64_t t) {
  const int64_t tiles = ((n + BN - 1) / BN) * ((t + BM - 1) / BM);
  const int cus = cu_count();
  int parts = 1;
  while (parts < 8 && tiles * parts * 2 <= cus && k % (256 * 2 * parts) == 0) parts *= 2;
  return parts;
}

hipError_t launch_gemm(int qtype, const void* w, int64_t n, int64_t k, const void* x, bool x_f32, int64_t t,
                       int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  return launch_gemm_split(qtype, w, n, k, x, x_f32, t, ldx, y, ldy, nullptr, 0, s);
}

hipError_t launch_gemm_split(int qtype, const void* w, int64_t n, int64_t k, const void* x, bool x_f32, int64_t t,
                             int64_t ldx, float* y, int64_t ldy, float* partial, int64_t partial_floats,
                             hipStream_t s) {
  GemmParams p = {};
  p.w = (const uint8_t*)w;
  p.rb = row_bytes_of(qtype, k);
  p.n = (int)n;
  p.k = (int)k;
  p.x = x;
  p.ldx = ldx;
  p.t = (int)t;
  p.y = y;
  p.ldy = ldy;
  p.vec_store = ldy % 4 == 0;
  if (!x_f32 && use_wide_tiles(qtype, kPlainF16, n, t, ldx, ldy)) return launch_gemm_wide(qtype, kPlainF16, 8, p, s);
  // Launches of half a round of 256 x 256 tiles (the 8B o and down at
  // T = 2048): measured per type, the producer-wave tall kernel below is the
  // fastest for Q6_K, Q4_K and Q5_K, whose decode it keeps off the MFMA
  // waves; Q2_K's cheap decode favours the wide kernel, in two K halves for
  // long K (down: 197 against 208 us) and with 128-token tiles otherwise (o:
  // 77 against 82 us).
  const bool q2_half_round = !x_f32 && qtype == kQ2_K && tall_strides_ok(ldx, ldy) &&
                             !wide_fills(((n + 255) / 256) * ((t + 255) / 256));
  if (q2_half_round && wide_halves_shape(n, k, t) && k >= 8192 && partial != nullptr && t * n <= partial_floats) {
    const int64_t cols = (n + wide_cols() - 1) / wide_cols();
    const int64_t kh = k / 2;
    p.seg.nseg = 2;
    for (int i = 0; i < 2; ++i) {
      p.seg.tile0[i] = (int)(i * cols);
      p.seg.w[i] = (const uint8_t*)w + i * row_bytes_of(qtype, kh);  // whole blocks: kh % 256 == 0
      p.seg.n[i] = (int)n;
      p.seg.k[i] = (int)kh;
      p.seg.xoff[i] = i * kh;
      p.seg.y[i] = i == 0 ? y : partial;
      p.seg.ldy[i] = i == 0 ? ldy : n;
    }
    for (int i = 2; i <= kMaxSeg; ++i) p.seg.tile0[i] = (int)(2 * cols);
    hipError_t e = launch_gemm_wide(qtype, kMulti, 8, p, s);
    if (e != hipSuccess) return e;
    const int64_t threads = t * ((n + 3) / 4);
    hipLaunchKernelGGL(add_partial_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s, partial, y, ldy,
                       (int)t, (int)n);
    return hipGetLastError();
  }
  if (q2_half_round && wide_fills(((n + 255) / 256) * ((t + 127) / 128))) return launch_gemm_wide(qtype, kPlainF16, 4, p, s);
  if (!x_f32 && use_tall_tiles(qtype, n, k, t, ldx, ldy)) {
    dim3 grid((uint32_t)((n + BN - 1) / BN), (uint32_t)((t + 255) / 256));
    return launch_gemm_tall(qtype, kPlainF16, grid, p, s);
  }
  if (!x_f32 && wide_supported(qtype, kPlainF16) && tall_strides_ok(ldx, ldy)) {
    int mi = 0, ks = 0;
    if (wide_ks_choice(n, k, t, mi, ks)) return launch_gemm_wide_ks(qtype, mi, ks, p, s);
  }
  const int parts = partial != nullptr ? gemm_ksplit_parts(n, k, t) : 1;
  if (parts > 1 && (int64_t)parts * t * n <= partial_floats) {
    // the parts write dense partial sums (row stride n, 16-byte rows when
    // n % 4 == 0), then one pass adds them in order into y
    p.k = (int)(k / parts);
    p.y = partial;
    p.ldy = n;
    p.part_stride = t * n;
    p.vec_store = n % 4 == 0;
    dim3 grid((uint32_t)((n + BN - 1) / BN), (uint32_t)((t + BM - 1) / BM), (uint32_t)parts);
    hipError_t e = x_f32 ? launch_mode<kPlainF32>(qtype, grid, p, s) : launch_mode<kPlainF16>(qtype, grid, p, s);
    if (e != hipSuccess) return e;
    const int64_t threads = t * ((n + 3) / 4);
    hipLaunchKernelGGL(ksplit_sum_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s, partial, t * n,
                       parts, y, ldy, (int)t, (int)n);
    return hipGetLastError();
  }
  dim3 grid((uint32_t)((n + BN - 1) / BN), (uint32_t)((t + BM - 1) / BM));
  return x_f32 ? launch_mode<kPlainF32>(qtype, grid, p, s) : launch_mode<kPlainF16>(qtype, grid, p, s);
}

// ---------------------------------------------------------------------------
// The K split without a caller workspace, for callers that cannot allocate:
// the partial sums go to `scratch`, a static device array that every GPU the
// library runs on holds until the process ends.  A split launch has
// tiles * parts < 2 * CUs (parts is the smallest power of two that reaches
// one workgroup per CU) and at most 128 x 128 outputs per tile, so on a GPU
// of up to 256 CUs its partial sums take under 512 * 16384 floats = 32 MiB.
// In host code `scratch` names a host-side stand-in: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gemm_noalloc(int qtype, const void* w, int64_t n, int64_t k, const void* x, bool x_f32, int64_t t,
                               int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  void* ptr = nullptr;
  hipError_t e = noalloc_scratch(&ptr);
  if (e != hipSuccess) return e;
  return launch_gemm_split(qtype, w, n, k, x, x_f32, t, ldx, y, ldy, (float*)ptr,
                           (int64_t)(kNoAllocScratchBytes / sizeof(float)), s);
}

// Per-head RMSNorm of y in place, for heads wider than the 128-column tile
// that the fused epilogue normalises within (head_dim 256): one wave per
// (token, head), lane l holding columns l, l + 64, ...; the same products as
// the epilogue (sum of squares, times 1 / head_dim, plus eps, v_rsq_f32, then
// value * scale * gain).
__global__ __launch_bounds__(256) void head_rmsnorm_kernel(float* __restrict__ y, int64_t ldy, int t, int n, int hd,
                                                           const float* __restrict__ gain, int64_t gstride, float eps) {
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int heads = n / hd;
  if (wid >= (int64_t)t * heads) return;
  const int tok = (int)(wid / heads), h = (int)(wid - (int64_t)tok * heads);
  const int lane = threadIdx.x & 63;
  float* row = y + (int64_t)tok * ldy + (int64_t)h * hd;
  const float* g = gain + (int64_t)h * gstride;
  float v[4];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = lane + 64 * e < hd ? row[lane + 64 * e] : 0.f;
    ss += v[e] * v[e];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float scale = __builtin_amdgcn_rsqf(ss * (1.f / (float)hd) + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (lane + 64 * e < hd) row[lane + 64 * e] = v[e] * scale * g[lane + 64 * e];
}

hipError_t launch_gemm_qknorm(int qtype, const void* w, int64_t n, int64_t k, const uint16_t* x, int64_t t,
                              int64_t ldx, int64_t head_dim, const float* gain, int64_t gain_head_stride,
                              float eps, float* y, int64_t ldy, hipStream_t s) {
  if (head_dim > 128) {
    // the projection, then the norm over each head of the stored rows
    hipError_t e = launch_gemm(qtype, w, n, k, x, false, t, ldx, y, ldy, s);
    if (e != hipSuccess || t == 0) return e;
    const int64_t waves = t * (n / head_dim);
    hipLaunchKernelGGL(head_rmsnorm_kernel, dim3((uint32_t)((waves + 3) / 4)), dim3(256), 0, s, y, ldy, (int)t, (int)n,
                       (int)head_dim, gain, gain_head_stride, eps);
    return hipGetLastError();
  }
  GemmParams p = {};
  p.w = (const uint8_t*)w;
  p.rb = row_bytes_of(qtype, k);
  p.n = (int)n;
  p.k = (int)k;
  p.x = x;
  p.ldx = ldx;
  p.t = (int)t;
  p.y = y;
  p.ldy = ldy;
  p.gain = gain;
  p.gstride = gain_head_stride;
  p.hd = (int)head_dim;
  p.eps = eps;
  p.vec_store = ldy % 4 == 0;
  if (use_tall_tiles(qtype, n, k, t, ldx, ldy)) {
    dim3 grid((uint32_t)((n + BN - 1) / BN), (uint32_t)((t + 255) / 256));
    return launch_gemm_tall(qtype, kQkNorm, grid, p, s);
  }
  dim3 grid((uint32_t)((n + BN - 1) / BN), (uint32_t)((t + BM - 1) / BM));
  return launch_mode<kQkNorm>(qtype, grid, p, s);
}

// The gate and up projections of a feed-forward layer over one X: one
// launch of the wide kernel with two segments where its tiles fill the GPU,
// else the two projections one after the other.
hipError_t launch_gemm_gate_up(int qtype, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                               const uint16_t* x, int64_t t, int64_t ldx, float* y_gate, int64_t ldy_gate, float* y_up,
                               int64_t ldy_up, hipStream_t s) {
  const int64_t cols = (n + wide_cols() - 1) / wide_cols();
  if (!wide_supported(qtype, kMulti) || !tall_strides_ok(ldx, ldy_gate) || !tall_strides_ok(ldx, ldy_up) ||
      !wide_fills(2 * cols * ((t + 255) / 256))) {
    hipError_t e = launch_gemm(qtype, w_gate, n, k, x, false, t, ldx, y_gate, ldy_gate, s);
    if (e != hipSuccess) return e;
    return launch_gemm(qtype, w_up, n, k, x, false, t, ldx, y_up, ldy_up, s);
  }
  GemmParams p = {};
  p.rb = row_bytes_of(qtype, k);
  p.k = (int)k;
  p.x = x;
  p.ldx = ldx;
  p.t = (int)t;
  p.seg.nseg = 2;
  const void* w[2] = {w_gate, w_up};
  float* y[2] = {y_gate, y_up};
  const int64_t ldy[2] = {ldy_gate, ldy_up};
  for (int i = 0; i < 2; ++i) {
    p.seg.tile0[i] = (int)(i * cols);
    p.seg.w[i] = (const uint8_t*)w[i];
    p.seg.n[i] = (int)n;
    p.seg.k[i] = (int)k;
    p.seg.y[i] = y[i];
    p.seg.ldy[i] = ldy[i];
  }
  for (int i = 2; i <= kMaxSeg; ++i) p.seg.tile0[i] = (int)(2 * cols);
  return launch_gemm_wide(qtype, kMulti, 8, p, s);
}

// Sums of the two K halves of split projections (k and v of the fused
// q/k/v launch), in that order: y = p0 + p1 (t x n, partials dense with row
// stride n, n % 8 == 0).  With hd > 0 the per-head RMSNorm follows, with the
// operations of the fused epilogue (sum of squares in f32, scale =
// rsq(ss * (1 / hd) + eps) with v_rsq_f32, then y * scale * gain).  One wave per (token, 512-column
// slab of its row); lane l holds columns 8 l .. 8 l + 7 of the slab, so a
// head (hd = 64 or 128) is hd / 8 adjacent lanes.  Both projections in one
// launch: the first one's waves, then the second one's.
struct SplitSum {
  const float* p0;
  const float* p1;
  float* y;
  int64_t ldy;
  int n, hd;
  const float* gain;
  int64_t gstride;
  int64_t items;  // waves: t * ceil(n / 512)
};

__global__ __launch_bounds__(256) void split_combine_kernel(SplitSum a, SplitSum b, float eps) {
  const int lane = threadIdx.x & 63;
  int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool first = item < a.items;
  const SplitSum& q = first ? a : b;
  if (!first) item -= a.items;
  if (item >= q.items) return;
  const int slabs = (q.n + 511) / 512;
  const int64_t tok = item / slabs;
  const int c = (int)(item - tok * slabs) * 512 + 8 * lane;
  const bool ok = c < q.n;  // n % 8 == 0: all 8 columns or none
  float4v lo = (float4v){0.f, 0.f, 0.f, 0.f}, hi = lo;
  if (ok) {
    const float4v* r0 = (const float4v*)(q.p0 + tok * q.n + c);
    const float4v* r1 = (const float4v*)(q.p1 + tok * q.n + c);
    // the two partial sums are read once
    lo = __builtin_nontemporal_load(r0) + __builtin_nontemporal_load(r1);
    hi = __builtin_nontemporal_load(r0 + 1) + __builtin_nontemporal_load(r1 + 1);
  }
  float4v* dst = (float4v*)(q.y + tok * q.ldy + c);
  if (q.hd == 0) {
    if (ok) {
      dst[0] = lo;
      dst[1] = hi;
    }
    return;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += lo[e] * lo[e] + hi[e] * hi[e];
  const int lanes = q.hd / 8;  // 8 or 16 lanes per head
  for (int m = 1; m < lanes; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float scale = __builtin_amdgcn_rsqf(ss * (1.f / (float)q.hd) + eps);
  if (ok) {
    const int head = c / q.hd;
    const float* g = q.gain + (int64_t)head * q.gstride + (c - head * q.hd);
    float4v o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = lo[e] * scale * g[e];
      o1[e] = hi[e] * scale * g[4 + e];
    }
    dst[0] = o0;
    dst[1] = o1;
  }
}


// Finish time of workgroups issued in order onto `slots` compute units, one
// at a time each (a tall tile takes a whole CU), with the given costs.
static double list_makespan(const std::vector<double>& cost, int slots) {
  std::vector<double> free_at((size_t)slots, 0.0);
  double end = 0.0;
  for (double c : cost) {
    const size_t best = (size_t)(std::min_element(free_at.begin(), free_at.end()) - free_at.begin());
    free_at[best] += c;
    end = std::max(end, free_at[best]);
  }
  return end;
}

int64_t qkv_split_partial_floats(const int64_t n[3], int64_t t) { return 2 * t * (n[1] + n[2]); }

// q, k and v over one X: when their output tiles together fill the GPU with
// tall tiles, one launch covers all three (each tile resolves its projection
// from its column index); otherwise three ordinary launches.
// In the fused launch the q tiles (largest projection, QK-norm epilogue) come
// first.  When the tiles fill the last round only in part and the caller gave
// room for partial sums, k and v are each split into two K halves (twice as
// many workgroups of half the work) that write partial sums; a combine pass
// then adds the halves in order and applies k's head norm.
hipError_t launch_gemm_qkv(int qtype, const void* const w[3], const int64_t n[3], int64_t k, const uint16_t* x,
                           int64_t t, int64_t ldx, int64_t head_dim, const float* const gain[3],
                           const int64_t gstride[3], float eps, float* const y[3], const int64_t ldy[3],
                           float* partial, hipStream_t s) {
  int64_t ntiles = 0;
  for (int i = 0; i < 3; ++i) ntiles += (n[i] + BN - 1) / BN;
  const int64_t mt = (t + 255) / 256;
  const bool fused = head_dim <= 128 && t >= 512 && ntiles * mt >= 256 && tall_weights_ok(qtype, k) &&
                     tall_strides_ok(ldx, ldy[0]) &&
                     tall_strides_ok(ldx, ldy[1]) && (n[2] == 0 || tall_strides_ok(ldx, ldy[2]));
  if (!fused) {
    for (int i = 0; i < 3; ++i) {
      if (n[i] == 0) continue;
      hipError_t e = i < 2 ? launch_gemm_qknorm(qtype, w[i], n[i], k, x, t, ldx, head_dim, gain[i], gstride[i], eps,
                                                y[i], ldy[i], s)
                           : launch_gemm(qtype, w[i], n[i], k, x, false, t, ldx, y[i], ldy[i], s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Split when the launch gets 10% shorter (halves start on a 256-weight
  // block: K % 512 == 0; the combine pass moves 8 floats per lane with
  // 16-byte accesses: n % 8 == 0 and 16-byte output rows).
  bool split = false;
  if (partial != nullptr && k % 512 == 0 && n[1] % 8 == 0 && n[2] % 8 == 0 && ldy[1] % 4 == 0 &&
      (n[2] == 0 || ldy[2] % 4 == 0)) {
    const int64_t cq = (n[0] + BN - 1) / BN, ckv = ntiles - cq;
    std::vector<double> whole((size_t)(ntiles * mt), 1.0), halves((size_t)(cq * mt), 1.0);
    halves.resize((size_t)((cq + 2 * ckv) * mt), 0.55);
    const int cus = cu_count();
    split = list_makespan(halves, cus) <= 0.9 * list_makespan(whole, cus);
  }
  GemmParams p = {};
  p.rb = row_bytes_of(qtype, k);
  p.k = (int)k;
  p.x = x;
  p.ldx = ldx;
  p.t = (int)t;
  p.hd = (int)head_dim;
  p.eps = eps;
  int nseg = 0, tile = 0;
  auto add_seg = [&](int i, int64_t k0, int64_t kk, float* out, int64_t ldo, int norm) {
    p.seg.tile0[nseg] = tile;
    p.seg.w[nseg] = (const uint8_t*)w[i] + row_bytes_of(qtype, k0);  // blocks before the K part
    p.seg.n[nseg] = (int)n[i];
    p.seg.k[nseg] = (int)kk;
    p.seg.xoff[nseg] = k0;
    p.seg.y[nseg] = out;
    p.seg.ldy[nseg] = ldo;
    p.seg.gain[nseg] = gain[i];
    p.seg.gstride[nseg] = gstride[i];
    p.seg.norm[nseg] = norm;
    tile += (int)((n[i] + BN - 1) / BN);
    ++nseg;
  };
  float* part[3][2] = {};
  float* next = partial;
  for (int i = 0; i < 3; ++i) {
    if (n[i] == 0) continue;
    if (split && i > 0) {
      for (int h = 0; h < 2; ++h) {
        part[i][h] = next;
        next += t * n[i];
        add_seg(i, h * (k / 2), k / 2, part[i][h], n[i], 0);
      }
    } else {
      add_seg(i, 0, k, y[i], ldy[i], i < 2);
    }
  }
  p.seg.nseg = nseg;
  for (int i = nseg; i <= kMaxSeg; ++i) p.seg.tile0[i] = tile;
  dim3 grid((uint32_t)mt, (uint32_t)tile);
  hipError_t e = launch_gemm_tall(qtype, kMulti, grid, p, s);
  if (e != hipSuccess || !split) return e;
  SplitSum sum[2] = {};
  for (int i = 1; i < 3; ++i) {
    SplitSum& q = sum[i - 1];
    if (n[i] == 0) continue;  // items 0: no waves
    q.p0 = part[i][0];
    q.p1 = part[i][1];
    q.y = y[i];
    q.ldy = ldy[i];
    q.n = (int)n[i];
    q.hd = i == 1 ? (int)head_dim : 0;
    q.gain = gain[i];
    q.gstride = gstride[i];
    q.items = t * ((n[i] + 511) / 512);
  }
  const int64_t waves = sum[0].items + sum[1].items;
  hipLaunchKernelGGL(split_combine_kernel, dim3((uint32_t)((waves + 3) / 4)), dim3(256), 0, s, sum[0], sum[1], eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Routed experts: router, token lists, combine.

// One wave per token: softmax over the experts, top_k by logit (largest
// first, ties to the lower index), weight = softmax probability.  Lane s
// keeps the s-th choice (top_k <= 64), so no register array is indexed at
// run time.  PER: slots of 64 experts (ne <= 64 PER).
template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int t, int ne, int top_k,
                                                         int renorm, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= t) return;
  float v[PER];
  const float* lg = logits + (int64_t)tok * ne;
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < ne ? lg[e] : -__builtin_inff();
    mx = __builtin_fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, 64));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < ne) sum += __expf(v[i] - mx);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
  uint32_t taken = 0;  // bit i: slot i of this lane already chosen
  float chosen = 0.f, my_w = 0.f;
  int my_id = 0;
  for (int s = 0; s < top_k; ++s) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < ne && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    const float w = __expf(bv - mx) / sum;
    chosen += w;
    if (lane == s) {
      my_w = w;
      my_id = bi;
    }
  }
  if (lane < top_k) {
    const float f = renorm ? 1.f / chosen : 1.f;
    ids[(int64_t)tok * top_k + lane] = my_id;
    weights[(int64_t)tok * top_k + lane] = my_w * f;
  }
}

hipError_t launch_route_topk(const float* logits, int64_t t, int64_t e, int64_t top_k, int renorm, int32_t* ids,
                             float* weights, hipStream_t s) {
  const dim3 grid((uint32_t)((t + 3) / 4));
  if (e <= 64)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, dim3(256), 0, s, logits, (int)t, (int)e, (int)top_k, renorm, ids,
                       weights);
  else if (e <= 128)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, dim3(256), 0, s, logits, (int)t, (int)e, (int)top_k, renorm, ids,
                       weights);
  else if (e <= 256)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, dim3(256), 0, s, logits, (int)t, (int)e, (int)top_k, renorm, ids,
                       weights);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, dim3(256), 0, s, logits, (int)t, (int)e, (int)top_k, renorm, ids,
                       weights);
  return hipGetLastError();
}

// Count the pairs of each expert (one workgroup per expert) and clear the
// row maxima of the h rows.
// Token lists of the routed experts, built chunk-parallel: chunk j holds
// pairs [256 j, 256 j + 256).  Histogram per chunk; per expert, an exclusive
// scan over its chunk counts; over experts, an exclusive scan of the totals;
// then a stable scatter (rank among the earlier pairs of the chunk with the
// same expert).  Each expert's list
// is therefore in pair order.  Ids outside [0, n_experts) are dropped and
// counted: per chunk here, summed into the workspace header by the offsets
// pass.
constexpr int kMoeChunk = 256;

__global__ __launch_bounds__(kMoeChunk) void moe_hist_kernel(const int32_t* __restrict__ ids, int npairs, int ne,
                                                             int nchunks, int* __restrict__ ccount,
                                                             int* __restrict__ cbad, uint32_t* __restrict__ rowmax) {
  __shared__ int hist[1024];
  __shared__ int bad;
  const int ch = blockIdx.x;
  for (int e = threadIdx.x; e < ne; e += kMoeChunk) hist[e] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int i = ch * kMoeChunk + threadIdx.x;
  if (i < npairs) {
    const int e = ids[i];
    if (e >= 0 && e < ne)
      atomicAdd(&hist[e], 1);
    else
      atomicAdd(&bad, 1);
    rowmax[i] = 0u;  // max |h| of compact row i, accumulated by the gate/up pass
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ne; e += kMoeChunk) ccount[(int64_t)e * nchunks + ch] = hist[e];
  if (threadIdx.x == 0) cbad[ch] = bad;
}

// Inclusive scan of v over the 1024 threads of a workgroup (wave shuffles,
// then the wave totals through LDS); returns the scan, *total the sum.
__device__ __forceinline__ int block_scan_1024(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int x = wsum[w];
    base += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();  // wsum may be rewritten by the next call
  *total = all;
  return v + base;
}

// One workgroup per expert: cpref[e][j] = pairs of expert e in chunks before j.
__global__ __launch_bounds__(1024) void moe_escan_kernel(const int* __restrict__ ccount, int nchunks,
                                                         int* __restrict__ cpref, int* __restrict__ counts) {
  __shared__ int wsum[16];
  const int64_t row = (int64_t)blockIdx.x * nchunks;
  int carry = 0;
  for (int b = 0; b < nchunks; b += 1024) {
    const int j = b + (int)threadIdx.x;
    const int v = j < nchunks ? ccount[row + j] : 0;
    int tot;
    const int incl = block_scan_1024(v, wsum, &tot);
    if (j < nchunks) cpref[row + j] = carry + incl - v;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = carry;
}

// One workgroup: first compact row of each expert (exclusive scan of the
// counts), the table of 128-row tiles per expert and the number of tiles;
// and the header's count of dropped pairs (the chunks' counts added in chunk
// order).
__global__ __launch_bounds__(1024) void moe_oscan_kernel(const int* __restrict__ counts, int ne,
                                                         int* __restrict__ offsets, int* __restrict__ tiles,
                                                         int* __restrict__ ntiles, int* __restrict__ tiles2,
                                                         int* __restrict__ ntiles2, int max_tiles2,
                                                         const int* __restrict__ cbad, int nchunks,
                                                         uint32_t* __restrict__ header) {
  __shared__ int wsum[16];
  {
    int nb = 0;
    for (int j = threadIdx.x; j < nchunks; j += 1024) nb += cbad[j];
    int tot;
    block_scan_1024(nb, wsum, &tot);
    if (threadIdx.x == 0) header[0] = (uint32_t)tot;
  }
  const int e = threadIdx.x;
  const int c = e < ne ? counts[e] : 0;
  const int nt = (c + BM - 1) / BM;
  // Tiles of the 256-row kernel as (expert, first row, rows, first compact
  // row of the tile: the expert's offset + first row).  The kernel
  // runs a tile of at most 128 rows over 4 M blocks and one of at most 192
  // over 6, so a list of 256 f + r rows with 0 < r <= 64 ends in tiles of
  // 192 and 64 + r rows rather than 256 and r (the weights are decoded once
  // per tile, whatever its rows).  Table order: tiles of more than 192
  // rows, then of 129-192, then of at most 128, so that the cheaper ones
  // fill the launch's last round.
  const int full = c / 256, rem = c % 256;
  const bool split = full >= 1 && rem > 0 && rem <= 64;
  const int n8 = split ? full - 1 : full + (rem > 192);
  const int n6 = split ? 1 : (rem > 128 && rem <= 192);
  const int n4 = split ? 1 : (rem > 0 && rem <= 128);
  int tot, tot8, tot6, tot4, rows_tot;
  const int cin = block_scan_1024(c, wsum, &rows_tot);
  const int tin8 = block_scan_1024(n8, wsum, &tot8);
  const int tin6 = block_scan_1024(n6, wsum, &tot6);
  const int tin4 = block_scan_1024(n4, wsum, &tot4);
  const int tin = block_scan_1024(nt, wsum, &tot);
  if (e < ne) {
    offsets[e] = cin - c;
    const int t0 = tin - nt;
    for (int k = 0; k < nt; ++k) {
      tiles[2 * (t0 + k)] = e;
      tiles[2 * (t0 + k) + 1] = k * BM;
    }
    auto put = [&](int u, int r0, int rows) {
      tiles2[4 * u] = e;
      tiles2[4 * u + 1] = r0;
      tiles2[4 * u + 2] = rows;
      tiles2[4 * u + 3] = cin - c + r0;
    };
    const int u8 = tin8 - n8;
    for (int k = 0; k < n8; ++k) put(u8 + k, 256 * k, min(256, c - 256 * k));
    if (n6) put(tot8 + tin6 - 1, 256 * n8, split ? 192 : rem);
    if (n4) put(tot8 + tot6 + tin4 - 1, split ? 256 * n8 + 192 : 256 * n8, split ? 64 + rem : rem);
  }
  if (e == 0) {
    ntiles[0] = tot;
    ntiles[1] = rows_tot;  // compact rows in all lists
    *ntiles2 = tot8 + tot6 + tot4;
  }
  // the rest of the 256-row table: tiles of no rows, which the kernel's
  // workgroups leave at once (so that they need not read the count first)
  for (int u = tot8 + tot6 + tot4 + threadIdx.x; u < max_tiles2; u += 1024) tiles2[4 * u + 2] = 0;
}

// Stable scatter: pair i of chunk j with expert e goes to compact row
// offsets[e] + cpref[e][j] + (number of earlier pairs of chunk j with expert e).
__global__ __launch_bounds__(kMoeChunk) void moe_scatter_kernel(const int32_t* __restrict__ ids, int npairs, int ne,
                                                                int nchunks, const int* __restrict__ offsets,
                                                                const int* __restrict__ cpref,
                                                                int* __restrict__ list) {
  __shared__ int sid[kMoeChunk];
  const int ch = blockIdx.x;
  const int i = ch * kMoeChunk + threadIdx.x;
  const int e = i < npairs ? ids[i] : -1;
  sid[threadIdx.x] = e;
  __syncthreads();
  if (e < 0 || e >= ne) return;
  int rank = 0;
  for (int j = 0; j < (int)threadIdx.x; ++j) rank += sid[j] == e;
  list[offsets[e] + cpref[(int64_t)e * nchunks + ch] + rank] = i;
}

// out[t, :] = sum over slots s (in order) of the weighted expert outputs of
// pair t * top_k + s; pairs with an id outside [0, n_experts) add nothing.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ dbuf, const int32_t* __restrict__ ids,
                                                          int t, int top_k, int ne, int hidden,
                                                          float* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of out
  const int64_t nq = (int64_t)t * hidden / 4;
  if (q >= nq) return;
  const int tok = (int)(q / (hidden / 4));
  const int c4 = (int)(q - (int64_t)tok * (hidden / 4));
  float4v acc = (float4v){0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < top_k; ++s) {
    const int64_t pair = (int64_t)tok * top_k + s;
    const int id = ids[pair];
    if (id < 0 || id >= ne) continue;
    const float4v v = *(const float4v*)(dbuf + pair * hidden + 4 * c4);
    acc += v;
  }
  *(float4v*)(out + (int64_t)tok * hidden + 4 * c4) = acc;
}

// Between the two passes of the 256-row kernel: per compact row, h =
// SiLU(g) * u = g / (1 + exp(-g)) * u (the same f32 products as the 128-row
// kernel's epilogue; SILU false: h itself from g, formed by the gate/up
// pass), the row's largest |h| (bits into pairmax at the row's pair), and h
// times
// the power of two that brings that maximum into [2^14, 2^15), rounded to
// binary16 (the down pass's A rows).  One wave per row; lane l holds columns
// 4 (l + 64 j) .. + 3, read and written 16 / 8 bytes at a time (inter is a
// multiple of 256, so of 4).
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

template <int NJ, bool SILU>
__global__ __launch_bounds__(256) void moe_silu_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                       const int* __restrict__ nrows, const int* __restrict__ list,
                                                       int inter, uint32_t* __restrict__ pairmax,
                                                       _Float16* __restrict__ h16) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= *nrows) return;
  const float* gr = g + (int64_t)row * inter;
  const float* ur = SILU ? u + (int64_t)row * inter : nullptr;
  float4v h[NJ];
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 4 * (lane + 64 * j);
    if (c < inter) {
      const float4v gv = SILU ? *(const float4v*)(gr + c) : __builtin_nontemporal_load((const float4v*)(gr + c));  // h: read once
      if constexpr (SILU) {
        const float4v uv = *(const float4v*)(ur + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) h[j][e] = gv[e] / (1.f + __expf(-gv[e])) * uv[e];
      } else {
        h[j] = gv;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(h[j][e]));
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, 64));
  const uint32_t bits = __builtin_bit_cast(uint32_t, mx);
  const float sc = row_scale_from_max(bits, false);
  if (lane == 0) pairmax[list[row]] = bits;  // by pair: the combine reads a token's slots in order
  _Float16* hr = h16 + (int64_t)row * inter;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 4 * (lane + 64 * j);
    if (c < inter) {
      const uint32_t lo = pack_f16x2(h[j][0] * sc, h[j][1] * sc), hi = pack_f16x2(h[j][2] * sc, h[j][3] * sc);
      *(uint2v*)(hr + c) = (uint2v){lo, hi};
    }
  }
}

// out[t, :] = sum over slots s (in order) of weights[t, s] * inverse scale *
// the down pass's row of pair t * top_k + s; pairs with an id outside
// [0, n_experts) add nothing.  The factor is the product the 128-row
// kernel's down epilogue applies, in the same order.  blockIdx.x is the
// token (its slot ids, maxima and weights are then uniform loads), thread i
// of blockIdx.y the float4 256 blockIdx.y + i of its row; the slots' rows are
// loaded 8 at a time before any is summed, so that 8 loads per thread are
// in flight, as non-temporal loads (each row is read once).
__global__ __launch_bounds__(256) void moe_combine_rows_kernel(const float* __restrict__ dbuf,
                                                               const int32_t* __restrict__ ids,
                                                               const uint32_t* __restrict__ pairmax,
                                                               const float* __restrict__ weights, int top_k, int ne,
                                                               int hidden, float* __restrict__ out) {
  const int tok = blockIdx.x;
  const int c4 = blockIdx.y * 256 + threadIdx.x;
  if (4 * c4 >= hidden) return;
  const int64_t pair0 = (int64_t)tok * top_k;
  const float* src = dbuf + pair0 * hidden + 4 * c4;
  float4v acc = (float4v){0.f, 0.f, 0.f, 0.f};
  // slots s0 .. s0 + 7 (past top_k: the last slot again, not summed)
  auto group = [&](int s0, auto whole) __attribute__((always_inline)) {
    int id[8];
    uint32_t mx[8];
    float wt[8];
    float4v v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = decltype(whole)::value ? s0 + j : min(s0 + j, top_k - 1);
      id[j] = ids[pair0 + s];
      mx[j] = pairmax[pair0 + s];
      wt[j] = weights[pair0 + s];
      v[j] = __builtin_nontemporal_load((const float4v*)(src + (int64_t)s * hidden));  // read once
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((decltype(whole)::value || s0 + j < top_k) && id[j] >= 0 && id[j] < ne)
        acc += v[j] * (row_scale_from_max(mx[j], true) * wt[j]);
  };
  int s0 = 0;
  for (; s0 + 8 <= top_k; s0 += 8) group(s0, std::true_type{});
  if (s0 < top_k) group(s0, std::false_type{});
  *(float4v*)(out + (int64_t)tok * hidden + 4 * c4) = acc;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool moe_workspace_layout(int64_t t, int64_t top_k, int64_t n_experts, int64_t hidden, int64_t inter,
                          MoeWorkspace& ws) {
  if (t < 0 || top_k <= 0 || n_experts <= 0 || hidden <= 0 || inter <= 0) return false;
  const int64_t pairs = t * top_k;
  ws.max_tiles = n_experts + (pairs + BM - 1) / BM;
  size_t o = 0;
  ws.nchunks = (pairs + kMoeChunk - 1) / kMoeChunk;
  ws.header = o;  o += 256;  // uint32 [0]: pairs dropped for an id outside [0, n_experts)
  ws.ccount = o;  o += align256(sizeof(int) * n_experts * ws.nchunks);
  ws.cbad = o;    o += align256(sizeof(int) * ws.nchunks);
  ws.cpref = o;   o += align256(sizeof(int) * n_experts * ws.nchunks);
  ws.counts = o;  o += align256(sizeof(int) * n_experts);
  ws.offsets = o; o += align256(sizeof(int) * n_experts);
  ws.max_tiles2 = (n_experts + (pairs + 255) / 256 + 7) / 8 * 8;  // whole groups of 8 (one per XCD)
  ws.ntiles = o;  o += align256(sizeof(int) * 4);
  ws.tiles = o;   o += align256(sizeof(int) * 2 * ws.max_tiles);
  ws.ntiles2 = o; o += align256(sizeof(int) * 4);
  ws.tiles2 = o;  o += align256(sizeof(int) * 4 * ws.max_tiles2);
  ws.list = o;    o += align256(sizeof(int) * pairs);
  ws.rowmax = o;  o += align256(sizeof(uint32_t) * pairs);
  ws.hbuf = o;    o += align256(sizeof(float) * pairs * inter);    // h (128-row kernel) or g (256-row kernel)
  ws.ubuf = o;    o += align256(sizeof(float) * pairs * inter);    // u (256-row kernel)
  ws.h16 = o;     o += align256(sizeof(uint16_t) * pairs * inter); // scaled binary16 h (256-row kernel)
  ws.dbuf = o;    o += align256(sizeof(float) * pairs * hidden);
  ws.total = o;
  return true;
}

hipError_t launch_grouped_expert(int qtype, const void* w_gate, const void* w_up, const void* w_down,
                                 int64_t n_experts, int64_t hidden, int64_t inter, const uint16_t* x, int64_t t,
                                 int64_t top_k, const int32_t* ids, const float* weights, float* out,
                                 void* workspace, const MoeWorkspace& ws, hipStream_t s) {
  char* wsb = (char*)workspace;
  int* counts = (int*)(wsb + ws.counts);
  int* offsets = (int*)(wsb + ws.offsets);
  int* ntiles = (int*)(wsb + ws.ntiles);
  int* tiles = (int*)(wsb + ws.tiles);
  int* list = (int*)(wsb + ws.list);
  uint32_t* rowmax = (uint32_t*)(wsb + ws.rowmax);
  float* hbuf = (float*)(wsb + ws.hbuf);
  float* dbuf = (float*)(wsb + ws.dbuf);
  const int npairs = (int)(t * top_k);
  hipError_t err;

  int* ccount = (int*)(wsb + ws.ccount);
  int* cbad = (int*)(wsb + ws.cbad);
  int* cpref = (int*)(wsb + ws.cpref);
  uint32_t* header = (uint32_t*)(wsb + ws.header);
  const int nch = (int)ws.nchunks;
  if (nch > 0) {
    hipLaunchKernelGGL(moe_hist_kernel, dim3((uint32_t)nch), dim3(kMoeChunk), 0, s, ids, npairs, (int)n_experts, nch,
                       ccount, cbad, rowmax);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(moe_escan_kernel, dim3((uint32_t)n_experts), dim3(1024), 0, s, ccount, nch, cpref, counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  int* ntiles2 = (int*)(wsb + ws.ntiles2);
  int* tiles2 = (int*)(wsb + ws.tiles2);
  // the 256-row kernel (the K-quant weight types) or the 128-row kernel
  const bool wide = wide_supported(qtype, kGrouped) && tall_strides_ok(hidden, inter) && tall_strides_ok(inter, hidden) &&
                    t * hidden * 2 < ((int64_t)1 << 31) &&  // gathered X rows: 32-bit byte offsets from x
                    inter <= 4096;                          // the SiLU pass holds a row in registers
  hipLaunchKernelGGL(moe_oscan_kernel, dim3(1), dim3(1024), 0, s, counts, (int)n_experts, offsets, tiles, ntiles,
                     tiles2, ntiles2, (int)ws.max_tiles2, cbad, nch, header);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (nch > 0) {
    hipLaunchKernelGGL(moe_scatter_kernel, dim3((uint32_t)nch), dim3(kMoeChunk), 0, s, ids, npairs, (int)n_experts,
                       nch, offsets, cpref, list);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (wide) {
    // gate and up: the tokens of each 256-row tile gathered through the list,
    // g and u into two f32 arrays of compact rows
    float* gbuf = (float*)(wsb + ws.hbuf);
    float* ubuf = (float*)(wsb + ws.ubuf);
    _Float16* h16 = (_Float16*)(wsb + ws.h16);
    const int64_t icols = (inter + 255) / 256, hcols = (hidden + 255) / 256;
    GemmParams p = {};
    p.tiles = tiles2;
    p.ntiles = ntiles2;
    p.offsets = offsets;
    p.counts = counts;
    p.list = list;
    p.top_k = (int)top_k;
    p.x = x;
    p.ldx = hidden;
    p.k = (int)hidden;
    p.rb = row_bytes_of(qtype, hidden);
    p.estride = p.rb * inter;
    p.t = (int)ws.max_tiles2;
    p.seg.nseg = 2;
    const uint8_t* wgu[2] = {(const uint8_t*)w_gate, (const uint8_t*)w_up};
    float* ygu[2] = {gbuf, ubuf};
    for (int i = 0; i < 2; ++i) {
      p.seg.tile0[i] = (int)(i * icols);
      p.seg.w[i] = wgu[i];
      p.seg.n[i] = (int)inter;
      p.seg.k[i] = (int)hidden;
      p.seg.y[i] = ygu[i];
      p.seg.ldy[i] = inter;
    }
    for (int i = 2; i <= kMaxSeg; ++i) p.seg.tile0[i] = (int)(2 * icols);
    // Q4_K / Q5_K with inter % 128 == 0: tiles of 128 gate and the same 128
    // up rows form h = SiLU(g) u themselves (gbuf), and the pass after
    // only scales h; otherwise g and u as two arrays and SiLU in that pass
    const bool fused = wide_supported(qtype, kGroupedGU) && inter % 128 == 0;
    if (fused) {
      GemmParams f = p;
      f.w = (const uint8_t*)w_gate;
      f.w2 = (const uint8_t*)w_up;
      f.n = (int)inter;
      f.y = gbuf;
      f.ldy = inter;
      if ((err = launch_gemm_wide(qtype, kGroupedGU, 8, f, s)) != hipSuccess) return err;
    } else if ((err = launch_gemm_wide(qtype, kGrouped, 8, p, s)) != hipSuccess) {
      return err;
    }
    {
      const dim3 g((uint32_t)((npairs + 3) / 4));
#define QP_SILU(NJ)                                                                                                 \
  if (fused)                                                                                                        \
    hipLaunchKernelGGL((moe_silu_kernel<NJ, false>), g, dim3(256), 0, s, gbuf, ubuf, ntiles + 1, list, (int)inter, \
                       rowmax, h16);                                                                                \
  else                                                                                                              \
    hipLaunchKernelGGL((moe_silu_kernel<NJ, true>), g, dim3(256), 0, s, gbuf, ubuf, ntiles + 1, list, (int)inter,  \
                       rowmax, h16);
      if (inter <= 1024) {
        QP_SILU(4)
      } else if (inter <= 2048) {
        QP_SILU(8)
      } else {
        QP_SILU(16)
      }
#undef QP_SILU
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // down: A = the binary16 h rows of each tile (compact rows, contiguous),
    // the raw products into dbuf's rows in pair order (row r of a tile goes
    // to pair list[r]), which the combine reads per token
    GemmParams d = p;
    // d.list stays: the epilogue stores row r of a tile at pair list[base + r]
    d.x = h16;
    d.ldx = inter;
    d.k = (int)inter;
    d.rb = row_bytes_of(qtype, inter);
    d.estride = d.rb * hidden;
    d.seg.nseg = 1;
    d.seg.tile0[0] = 0;
    d.seg.w[0] = (const uint8_t*)w_down;
    d.seg.n[0] = (int)hidden;
    d.seg.k[0] = (int)inter;
    d.seg.y[0] = dbuf;
    d.seg.ldy[0] = hidden;
    for (int i = 1; i <= kMaxSeg; ++i) d.seg.tile0[i] = (int)hcols;
    if ((err = launch_gemm_wide(qtype, kGroupedDown, 8, d, s)) != hipSuccess) return err;
    if (t == 0) return hipSuccess;
    hipLaunchKernelGGL(moe_combine_rows_kernel, dim3((uint32_t)t, (uint32_t)((hidden / 4 + 255) / 256)), dim3(256), 0, s,
                       dbuf, ids, rowmax, weights, (int)top_k, (int)n_experts, (int)hidden, out);
    return hipGetLastError();
  }

  GemmParams p = {};
  p.tiles = tiles;
  p.ntiles = ntiles;
  p.offsets = offsets;
  p.counts = counts;
  p.list = list;
  p.top_k = (int)top_k;
  p.rowmax = rowmax;
  p.hbuf = hbuf;
  p.dbuf = dbuf;
  p.weights = weights;
  p.vec_store = inter % 4 == 0 && hidden % 4 == 0;  // h and expert-output rows of 16-byte multiples

  // gate/up: A = gathered token rows, W tile = 64 gate rows + 64 up rows
  p.w = (const uint8_t*)w_gate;
  p.w2 = (const uint8_t*)w_up;
  p.rb = row_bytes_of(qtype, hidden);
  p.estride = p.rb * inter;
  p.n = (int)inter;
  p.k = (int)hidden;
  p.x = x;
  p.ldx = hidden;
  dim3 g1((uint32_t)ws.max_tiles, (uint32_t)((inter + BN / 2 - 1) / (BN / 2)));
  if ((err = launch_mode<kGateUp>(qtype, g1, p, s)) != hipSuccess) return err;

  // down: A = h rows (scaled to binary16 per row), weighted scatter to dbuf
  p.w = (const uint8_t*)w_down;
  p.w2 = nullptr;
  p.rb = row_bytes_of(qtype, inter);
  p.estride = p.rb * hidden;
  p.n = (int)hidden;
  p.k = (int)inter;
  p.x = nullptr;
  dim3 g2((uint32_t)ws.max_tiles, (uint32_t)((hidden + BN - 1) / BN));
  if ((err = launch_mode<kDown>(qtype, g2, p, s)) != hipSuccess) return err;

  const int64_t nq = t * hidden / 4;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((uint32_t)((nq + 255) / 256)), dim3(256), 0, s, dbuf, ids, (int)t,
                     (int)top_k, (int)n_experts, (int)hidden, out);
  return hipGetLastError();
}

}  // namespace qp
