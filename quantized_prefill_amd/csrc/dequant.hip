// dequant.hip -- streaming dequant of a GGUF block-quantized tensor to f32 or
// binary16 ("Qwen3.5 batched prefill has no f32 dequant for IQ2_XXS, IQ3_S,
// IQ3_XXS, Q2_K", sections "Cause" and "Acceptance (each row)": bit-exact f32
// dequant, the f16 copy built from the f32 value, a partial last block
// handled, nothing written outside the output).
//
// HBM-bound: per weight the kernel reads type_size/QK bytes and writes 4
// (f32) or 2 (f16) bytes, so the design is about the write stream.
//
// Dense tensors (cols a multiple of QK, the case of every model projection):
// the output is the flat sequence of block values, so each lane owns V
// consecutive outputs (V = 4 floats or 8 halfs, one 16-byte store) and one
// store instruction of a wave writes 1 KB of contiguous output.  Each lane
// reads only the few bytes of its V weights (quants, scale, d), which the
// wave's lanes fetch from the same one or two blocks.  A wave handles G such
// groups, issuing all loads before the first store; G = 1 measured fastest
// (the HBM write stream wants many short-lived waves).
//
// Partial last blocks (cols % QK != 0): one thread decodes one unit (32
// consecutive weights of a block).  Rows of the tensor are whole blocks back
// to back, so block g of the flat block sequence is block g % nb of row
// g / nb; only the cols valid weights of each row are stored.
#include "qp_device.h"
#include "qp_internal.h"

namespace qp {

template <int QT, bool F16OUT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ src, uint32_t nb,
                                                      int64_t cols, uint64_t total_units,
                                                      void* __restrict__ dst_) {
  using F = Fmt<QT>;
  const uint64_t unit = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (unit >= total_units) return;
  const uint64_t g = unit / (uint32_t)F::UNITS;  // flat block index
  const uint32_t u = (uint32_t)(unit % (uint32_t)F::UNITS);
  const uint64_t r = g / nb;
  const uint32_t bi = (uint32_t)(g - r * nb);
  const int64_t c0 = (int64_t)bi * F::QK + 32 * (int64_t)u;
  if (c0 >= cols) return;  // unused quants of a partial last block
  const int64_t valid64 = cols - c0;
  const int valid = valid64 < 32 ? (int)valid64 : 32;

  UnitRaw raw;
  load_unit<QT>(src + g * F::TS, u, raw);
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = unit_value_exact<QT>(raw, i);

  const int64_t off = (int64_t)r * cols + c0;
  if constexpr (!F16OUT) {
    float* o = (float*)dst_ + off;
    if (valid == 32 && ((uintptr_t)o & 15) == 0) {
      float4v* o4 = (float4v*)o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o4[j] = (float4v){v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (i < valid) o[i] = v[i];
    }
  } else {
    uint16_t* o = (uint16_t*)dst_ + off;
    if (valid == 32 && ((uintptr_t)o & 15) == 0) {
      u32x4* o4 = (u32x4*)o;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o4[j] = (u32x4){pack_f16x2(v[8 * j], v[8 * j + 1]), pack_f16x2(v[8 * j + 2], v[8 * j + 3]),
                        pack_f16x2(v[8 * j + 4], v[8 * j + 5]), pack_f16x2(v[8 * j + 6], v[8 * j + 7])};
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (i < valid) o[i] = f32_to_f16_bits(v[i]);
    }
  }
}

template <int QT, bool F16OUT, int G>
__global__ __launch_bounds__(256) void dequant_flat_kernel(const uint8_t* __restrict__ src, uint64_t total,
                                                           void* __restrict__ dst_) {
  using F = Fmt<QT>;
  constexpr int V = F16OUT ? 8 : 4;
  constexpr uint64_t GW = 64 * V;  // weights per wave group
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63;
  Span<QT, V> sp[G];
  uint64_t w0[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    w0[g] = (wave * G + g) * GW + (uint64_t)lane * V;
    if (w0[g] < total) sp[g].load(src + (w0[g] / F::QK) * F::TS, (uint32_t)(w0[g] % F::QK));
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (w0[g] >= total) continue;
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = sp[g].value(i);
    if constexpr (!F16OUT) {
      __builtin_nontemporal_store((float4v){v[0], v[1], v[2], v[3]}, (float4v*)((float*)dst_ + w0[g]));
    } else {
      __builtin_nontemporal_store((u32x4){pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
                                          pack_f16x2(v[6], v[7])},
                                  (u32x4*)((uint16_t*)dst_ + w0[g]));
    }
  }
}

// F16 weights (one binary16 per weight): the f32 output is the exact
// widening, the f16 output the nearest-even binary16 of that f32 value (the
// same bits, NaN payloads aside).  A thread owns 8 consecutive weights: one
// 16-byte load and 16-byte stores where the run is whole and aligned, else
// element by element.
template <bool F16OUT>
__global__ __launch_bounds__(256) void dequant_f16w_kernel(const uint16_t* __restrict__ src, uint64_t total,
                                                           void* __restrict__ dst_) {
  const uint64_t i0 = 8 * ((uint64_t)blockIdx.x * 256u + threadIdx.x);
  if (i0 >= total) return;
  const bool vec = i0 + 8 <= total && (((uintptr_t)dst_ | (uintptr_t)src) & 15) == 0;
  if (vec) {
    const u32x4 v = *(const u32x4*)(src + i0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = f16_to_f32(w[j] & 0xFFFFu);
      f[2 * j + 1] = f16_to_f32(w[j] >> 16);
    }
    if constexpr (!F16OUT) {
      float4v* o = (float4v*)((float*)dst_ + i0);
      __builtin_nontemporal_store((float4v){f[0], f[1], f[2], f[3]}, o);
      __builtin_nontemporal_store((float4v){f[4], f[5], f[6], f[7]}, o + 1);
    } else {
      __builtin_nontemporal_store((u32x4){pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]), pack_f16x2(f[4], f[5]),
                                          pack_f16x2(f[6], f[7])},
                                  (u32x4*)((uint16_t*)dst_ + i0));
    }
    return;
  }
  const uint64_t n = total - i0 < 8 ? total - i0 : 8;
  for (uint64_t j = 0; j < n; ++j) {
    const float f = f16_to_f32(src[i0 + j]);
    if constexpr (!F16OUT)
      ((float*)dst_)[i0 + j] = f;
    else
      ((uint16_t*)dst_)[i0 + j] = f32_to_f16_bits(f);
  }
}

template <int QT, bool F16OUT>
static hipError_t launch_dequant_t(const void* src, int64_t rows, int64_t cols, void* dst, hipStream_t s) {
  using F = Fmt<QT>;
  if (cols % F::QK == 0 && ((uintptr_t)dst & 15) == 0) {
    constexpr int G = 1;  // one group per wave: more waves in flight beat more stores per wave
    const uint64_t total = (uint64_t)rows * cols;
    const uint64_t gw = F16OUT ? 512 : 256;
    const uint64_t waves = ((total + gw - 1) / gw + G - 1) / G;
    hipLaunchKernelGGL((dequant_flat_kernel<QT, F16OUT, G>), dim3((uint32_t)((waves + 3) / 4)), dim3(256), 0, s,
                       (const uint8_t*)src, total, dst);
    return hipGetLastError();
  }
  const uint32_t nb = (uint32_t)((cols + F::QK - 1) / F::QK);
  const uint64_t units = (uint64_t)rows * nb * F::UNITS;
  const uint64_t grid = (units + 255) / 256;
  hipLaunchKernelGGL((dequant_kernel<QT, F16OUT>), dim3((uint32_t)grid), dim3(256), 0, s,
                     (const uint8_t*)src, nb, cols, units, dst);
  return hipGetLastError();
}

hipError_t launch_dequant(int qtype, bool f16out, const void* src, int64_t rows, int64_t cols, void* dst,
                          hipStream_t s) {
  switch (qtype) {
    case kF16: {
      const uint64_t total = (uint64_t)rows * cols;
      const dim3 grid((uint32_t)((total + 8 * 256 - 1) / (8 * 256)));
      if (f16out)
        hipLaunchKernelGGL(dequant_f16w_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)src, total, dst);
      else
        hipLaunchKernelGGL(dequant_f16w_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)src, total, dst);
      return hipGetLastError();
    }
    case kQ8_0: return f16out ? launch_dequant_t<kQ8_0, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ8_0, false>(src, rows, cols, dst, s);
    case kQ4_K: return f16out ? launch_dequant_t<kQ4_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ4_K, false>(src, rows, cols, dst, s);
    case kQ5_K: return f16out ? launch_dequant_t<kQ5_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ5_K, false>(src, rows, cols, dst, s);
    case kQ6_K: return f16out ? launch_dequant_t<kQ6_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ6_K, false>(src, rows, cols, dst, s);
    case kQ2_K: return f16out ? launch_dequant_t<kQ2_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ2_K, false>(src, rows, cols, dst, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qp
