// dequant.hip -- streaming dequant of a GGUF block-quantized tensor to f32 or
// binary16 ("Qwen3.5 batched prefill has no f32 dequant for IQ2_XXS, IQ3_S,
// IQ3_XXS, Q2_K", sections "Cause" and "Acceptance (each row)": bit-exact f32
// dequant, the f16 copy built from the f32 value, a partial last block
// handled, nothing written outside the output).
//
// One thread decodes one unit (32 consecutive weights of a block).  Rows of
// the tensor are whole blocks back to back, so block g of the flat block
// sequence is block g % nb of row g / nb.  Adjacent lanes take adjacent
// units, so a wave's block fields come from a few cache lines and its 16-byte
// stores cover a contiguous run of the output.  HBM-bound: per weight the
// kernel reads type_size/QK bytes and writes 4 (f32) or 2 (f16) bytes.
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

template <int QT, bool F16OUT>
static hipError_t launch_dequant_t(const void* src, int64_t rows, int64_t cols, void* dst, hipStream_t s) {
  using F = Fmt<QT>;
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
    case kQ8_0: return f16out ? launch_dequant_t<kQ8_0, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ8_0, false>(src, rows, cols, dst, s);
    case kQ4_K: return f16out ? launch_dequant_t<kQ4_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ4_K, false>(src, rows, cols, dst, s);
    case kQ6_K: return f16out ? launch_dequant_t<kQ6_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ6_K, false>(src, rows, cols, dst, s);
    case kQ2_K: return f16out ? launch_dequant_t<kQ2_K, true>(src, rows, cols, dst, s)
                              : launch_dequant_t<kQ2_K, false>(src, rows, cols, dst, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qp
