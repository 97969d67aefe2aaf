// kv.hip -- the two steps between the attention-input projections and the
// prompt attention: the rotary position step on the QK-normed Q and K rows,
// and the write of the chunk's K and V rows into the KV cache held as
// binary16, Q8_0 ("INT8") or Q4_0 rows ("CUDA prefill VRAM loans and SM75
// Q4/native-IQ opt-ins", section "Summary" and the KV table after it).
//
// Both are small elementwise passes (T x heads x head_dim values), bound by
// HBM latency rather than bandwidth at prefill sizes; they stay separate
// kernels so that the projections and the attention keep their own tiles.
#include "qp_device.h"
#include "qp_internal.h"

namespace qp {

// Rotary step, half-split pairs: values j and j + head_dim/2 of each head of
// row i turn by (pos0 + i) * base^(-2j / head_dim).  One thread per (row,
// pair) computes the angle, cosine and sine in binary64 once and applies
// them to that pair of every head; each result is rounded to f32 once.
// (Positions reach 10^5 and more: an f32 angle would lose the low bits that
// decide the rotation.)
__global__ __launch_bounds__(256) void rope_kernel(float* __restrict__ x, int64_t ldx, int t, int n_head, int hd,
                                                   int64_t pos0, double base) {
  const int half = hd >> 1;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)t * half) return;
  const int i = (int)(idx / half), j = (int)(idx - (int64_t)i * half);
  const double inv_freq = pow(base, -2.0 * (double)j / (double)hd);
  const double theta = (double)(pos0 + i) * inv_freq;
  double sn, c;
  sincos(theta, &sn, &c);
  float* row = x + (int64_t)i * ldx + j;
  for (int h = 0; h < n_head; ++h) {
    float* v = row + (int64_t)h * hd;
    const double a = (double)v[0], b = (double)v[half];
    v[0] = (float)(a * c - b * sn);
    v[half] = (float)(a * sn + b * c);
  }
}

hipError_t launch_rope(float* x, int64_t ldx, int64_t t, int64_t n_head, int64_t head_dim, int64_t pos0, double base,
                       hipStream_t s) {
  const int64_t threads = t * (head_dim / 2);
  hipLaunchKernelGGL(rope_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s, x, ldx, (int)t,
                     (int)n_head, (int)head_dim, pos0, base);
  return hipGetLastError();
}

// KV cache rows.  Thread b takes 32 consecutive values of one (token, kv
// head): block c of cache row (row0 + i) * n_kv + g.  The quantizers are the
// GGUF reference rounding in binary32 (contraction off: no fused
// multiply-add may change a code):
//   Q8_0  d = amax / 127, code = round-half-away(x * (1 / d)) (0 when d = 0)
//   Q4_0  d = m / -8 for m the first value of largest magnitude,
//         code = min(15, trunc(x * (1 / d) + 8.5)), values 16..31 in the high nibbles
//   F16   the nearest-even binary16 of each value
// and each block stores the nearest-even binary16 of its f32 d.
// d is passed through an empty asm statement before its conversion: the
// compiler would otherwise fold d = m * -0.125 and the rounding to binary16
// into one fma_mix with a +0 addend, which turns d = -0 into +0.
__device__ __forceinline__ uint16_t scale_bits(float d) {
  asm volatile("" : "+v"(d));
  return f32_to_f16_bits(d);
}

template <int KV>
__global__ __launch_bounds__(256) void kv_write_kernel(const float* __restrict__ src, int64_t lds, int t, int n_kv,
                                                       int hd, uint8_t* __restrict__ cache, int64_t row0) {
#pragma clang fp contract(off)  // x * (1 / d) + 8.5 is two roundings, never one fma (the
                                // pragma covers the operators written here, not called helpers)
  const int bpr = hd / 32;  // 32-value blocks per head row
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= (int64_t)t * n_kv * bpr) return;
  const int c = (int)(b % bpr);
  const int64_t r = b / bpr;  // chunk row: token i, kv head g
  const int i = (int)(r / n_kv), g = (int)(r - (int64_t)i * n_kv);
  const float* x = src + (int64_t)i * lds + (int64_t)g * hd + 32 * c;
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; e += 4) {
    const float4v q = *(const float4v*)(x + e);
    v[e] = q[0];
    v[e + 1] = q[1];
    v[e + 2] = q[2];
    v[e + 3] = q[3];
  }
  const int64_t crow = (row0 + i) * n_kv + g;
  if constexpr (KV == kF16) {
    uint32_t* o = (uint32_t*)(cache + crow * (int64_t)hd * 2 + 64 * c);
#pragma unroll
    for (int e = 0; e < 32; e += 2) o[e / 2] = pack_f16x2(v[e], v[e + 1]);
  } else if constexpr (KV == kQ8_0) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    const float d = amax / 127.0f;
    const float id = d != 0.f ? 1.0f / d : 0.f;
    uint16_t* o = (uint16_t*)(cache + crow * (int64_t)bpr * 34 + 34 * c);
    o[0] = scale_bits(d);
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      const int q0 = (int)roundf(v[e] * id), q1 = (int)roundf(v[e + 1] * id);
      o[1 + e / 2] = (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
    }
  } else {  // Q4_0
    float amax = 0.f, m = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float a = fabsf(v[e]);
      if (a > amax) {
        amax = a;
        m = v[e];
      }
    }
    const float d = m / -8.0f;
    const float id = d != 0.f ? 1.0f / d : 0.f;
    int q[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float p = v[e] * id;  // rounded here: contraction is off in this kernel
      const int k = (int)(p + 8.5f);
      q[e] = k > 15 ? 15 : k;
    }
    uint16_t* o = (uint16_t*)(cache + crow * (int64_t)bpr * 18 + 18 * c);
    o[0] = scale_bits(d);
#pragma unroll
    for (int e = 0; e < 16; e += 2)
      o[1 + e / 2] = (uint16_t)((q[e] | (q[e + 16] << 4)) | ((q[e + 1] | (q[e + 17] << 4)) << 8));
  }
}

hipError_t launch_kv_write(int kv_type, const float* src, int64_t lds, int64_t t, int64_t n_kv, int64_t head_dim,
                           void* cache, int64_t row0, hipStream_t s) {
  const int64_t blocks = t * n_kv * (head_dim / 32);
  const dim3 grid((uint32_t)((blocks + 255) / 256));
  uint8_t* c = (uint8_t*)cache;
  switch (kv_type) {
    case kF16:
      hipLaunchKernelGGL(kv_write_kernel<kF16>, grid, dim3(256), 0, s, src, lds, (int)t, (int)n_kv, (int)head_dim, c,
                         row0);
      break;
    case kQ8_0:
      hipLaunchKernelGGL(kv_write_kernel<kQ8_0>, grid, dim3(256), 0, s, src, lds, (int)t, (int)n_kv, (int)head_dim, c,
                         row0);
      break;
    case kQ4_0:
      hipLaunchKernelGGL(kv_write_kernel<kQ4_0>, grid, dim3(256), 0, s, src, lds, (int)t, (int)n_kv, (int)head_dim, c,
                         row0);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qp
