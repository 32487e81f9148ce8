// mx_kernels.hip -- gfx950 kernels for block-shared-exponent quantization.
//
// Generic layout: one lane owns one 32-value block.  The lane reads the
// block (64 B of bf16 or 128 B of fp32) with 128-bit loads, reduces the
// largest magnitude in registers, derives the shared scale, rounds every
// value, and writes its packed codes (24/16/32 B) and its scale byte.  No
// value crosses lanes, so every output byte has exactly one writer.
//
// Rules: "Online MXFP6" page ("Start a model": packed codes and an E8M0
// scale per 32 values); "EFQ-Softmax" explainer (exponent-only block scale
// from the block's local maximum; exp-then-quantize); "AXS-6" page
// ("Overview" block layout; "Quick Start" fused fake-quantize).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_formats.h"
#include "mx_kernels.h"

namespace mxk {

// ---------------------------------------------------------------------------
// Loading one block into 32 fp32 bit patterns.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load_block(const void* x, int64_t b, uint32_t (&v)[32]) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(x) + b * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 q = p[i];
      uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = w[j] << 16;
        v[8 * i + 2 * j + 1] = w[j] & 0xFFFF0000u;
      }
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(x) + b * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 q = p[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
}

// Storing 32 output values given as fp32 bit patterns (bf16: rounded).
template <bool BF16>
__device__ __forceinline__ void store_block(void* y, int64_t b, const uint32_t (&v)[32]) {
  if constexpr (BF16) {
    uint4* p = reinterpret_cast<uint4*>(y) + b * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = f32_to_bf16_rne(__uint_as_float(v[8 * i + 2 * j])) |
               (f32_to_bf16_rne(__uint_as_float(v[8 * i + 2 * j + 1])) << 16);
      p[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    uint4* p = reinterpret_cast<uint4*>(y) + b * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

template <int W>
__device__ __forceinline__ void store_codes(void* codes, int64_t b, const uint32_t (&o)[W]) {
  if constexpr (W == 6) {
    uint2* p = reinterpret_cast<uint2*>(codes) + b * 3;
    p[0] = make_uint2(o[0], o[1]);
    p[1] = make_uint2(o[2], o[3]);
    p[2] = make_uint2(o[4], o[5]);
  } else if constexpr (W == 4) {
    uint4* p = reinterpret_cast<uint4*>(codes) + b;
    p[0] = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    uint4* p = reinterpret_cast<uint4*>(codes) + b * 2;
    p[0] = make_uint4(o[0], o[1], o[2], o[3]);
    p[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

template <int W>
__device__ __forceinline__ void load_codes(const void* codes, int64_t b, uint32_t (&o)[W]) {
  if constexpr (W == 6) {
    const uint2* p = reinterpret_cast<const uint2*>(codes) + b * 3;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      uint2 q = p[i];
      o[2 * i] = q.x;
      o[2 * i + 1] = q.y;
    }
  } else if constexpr (W == 4) {
    uint4 q = reinterpret_cast<const uint4*>(codes)[b];
    o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(codes) + b * 2;
    uint4 q0 = p[0], q1 = p[1];
    o[0] = q0.x; o[1] = q0.y; o[2] = q0.z; o[3] = q0.w;
    o[4] = q1.x; o[5] = q1.y; o[6] = q1.z; o[7] = q1.w;
  }
}

// ---------------------------------------------------------------------------
// One block in registers: scale byte and codes (the quantize core).
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ uint32_t quantize_regs(const uint32_t (&v)[32], uint32_t (&c)[32],
                                                  float (&r)[32]) {
  using T = Fmt<F>;
  uint32_t amax = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = max(amax, v[k] & 0x7FFFFFFFu);
  const uint32_t byte = scale_byte_from_amax<F>(amax);
  const int neg_exp = 127 - (int)byte;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    Rounded q = round_scaled<F>(scaled_abs<F>(v[k], neg_exp));
    const uint32_t sign = v[k] >> 31;
    c[k] = (byte == 0xFFu) ? 0u : (q.mag | (sign << (T::W - 1)));
    r[k] = q.val;
  }
  return byte;
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <int F, bool BF16>
__global__ __launch_bounds__(256) void quantize_lpb(const void* __restrict__ x, int64_t nb,
                                                    void* __restrict__ codes,
                                                    uint8_t* __restrict__ scales,
                                                    uint8_t* __restrict__ aux) {
  constexpr int W = Fmt<F>::W;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    uint32_t v[32], c[32], o[W];
    float r[32];
    load_block<BF16>(x, b, v);
    const uint32_t byte = quantize_regs<F>(v, c, r);
    pack32<W>(c, o);
    store_codes<W>(codes, b, o);
    scales[b] = (uint8_t)byte;
    // AXS-6 config plane: 2 bits per block, all zero (the uniform grid)
    if constexpr (F == F_AXS6) {
      if ((b & 3) == 0) aux[b >> 2] = 0;
    }
  }
}

template <int F, bool BF16>
__global__ __launch_bounds__(256) void fake_quantize_lpb(const void* x, int64_t nb, void* y) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    uint32_t v[32], c[32], out[32];
    float r[32];
    load_block<BF16>(x, b, v);
    const uint32_t byte = quantize_regs<F>(v, c, r);
    const int sexp = (int)byte - 127;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float mag = __builtin_ldexpf(r[k], sexp);
      out[k] = (byte == 0xFFu) ? 0x7FC00000u : (__float_as_uint(mag) | (v[k] & 0x80000000u));
    }
    store_block<BF16>(y, b, out);
  }
}

template <int F, bool BF16>
__global__ __launch_bounds__(256) void dequantize_lpb(const void* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ aux, int64_t nb,
                                                      void* __restrict__ y) {
  using T = Fmt<F>;
  constexpr int W = T::W;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    uint32_t o[W], out[32];
    load_codes<W>(codes, b, o);
    const uint32_t byte = scales[b];
    bool poisoned = (byte == 0xFFu);
    if constexpr (F == F_AXS6) poisoned |= ((aux[b >> 2] >> (2 * (b & 3))) & 3u) != 0u;
    const int sexp = (int)byte - 127;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t code = unpack1<W>(o, k);
      const uint32_t mag = code & ((1u << (W - 1)) - 1u);
      const uint32_t sign = (code >> (W - 1)) << 31;
      const float val = decode_mag<F>(mag, sexp);
      bool nan = poisoned;
      if constexpr (T::NAN_MAG >= 0) nan |= (mag == (uint32_t)T::NAN_MAG);
      out[k] = nan ? 0x7FC00000u : (__float_as_uint(val) | sign);
    }
    store_block<BF16>(y, b, out);
  }
}

// ---------------------------------------------------------------------------
// Exp-then-quantize probabilities: one wavefront per row.
// exp_fixed is the fp32 op sequence of the library's contract: Cody-Waite
// reduction (Cody and Waite, "Software Manual for the Elementary
// Functions", 1980) with ln2 split into a 16-bit head and a tail, a degree-7
// Taylor polynomial by Horner's rule with fused multiply-adds, and scaling by
// exact power-of-two products.  Constants: log2(e), ln2 and 1/k! rounded to
// fp32; head = ln2's fp32 significand cut to 16 bits, tail = fp32(ln2 - head).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_fixed(float d) {
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.62e400p-1f;
  const float kLn2Lo = 0x1.7f7d1cp-20f;
  const float k2 = 0x1.000000p-1f, k3 = 0x1.555556p-3f, k4 = 0x1.555556p-5f,
              k5 = 0x1.111112p-7f, k6 = 0x1.6c16c2p-10f, k7 = 0x1.a01a02p-13f;
  // the reduction runs on d clamped into [-104, 88.75] (NaN -> -104) so the
  // integer n stays in range; the selects below handle the outside
  const float dc = fminf(fmaxf(d, -104.0f), 88.75f);
  const float nf = __builtin_rintf(dc * kLog2e);
  float r = __builtin_fmaf(-nf, kLn2Hi, dc);
  r = __builtin_fmaf(-nf, kLn2Lo, r);
  float p = k7;
  p = __builtin_fmaf(p, r, k6);
  p = __builtin_fmaf(p, r, k5);
  p = __builtin_fmaf(p, r, k4);
  p = __builtin_fmaf(p, r, k3);
  p = __builtin_fmaf(p, r, k2);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  int n = (int)nf;
  if (n < -100) { p = p * 0x1p-50f; n += 50; }
  if (n > 100) { p = p * 0x1p+50f; n -= 50; }
  float res = p * __uint_as_float((uint32_t)(n + 127) << 23);
  // outside the reduction's range: below -104 the result rounds to +0,
  // above 88.75 it overflows; NaN propagates
  res = (d < -104.0f) ? 0.0f : res;
  res = (d > 88.75f) ? __builtin_inff() : res;
  res = (d != d) ? d : res;
  return res;
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  return m;
}

__device__ __forceinline__ int wave_or(int f) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) f |= __shfl_xor(f, off, 64);
  return f;
}

template <int F>
__global__ __launch_bounds__(256) void softmax_quantize_rows(const float* __restrict__ s,
                                                             int64_t rows, int64_t cols,
                                                             void* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  constexpr int W = Fmt<F>::W;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t nbr = cols >> 5;
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); row < rows;
       row += waves) {
    const float* srow = s + row * cols;
    // pass 1: exact row maximum (NaN anywhere makes it NaN)
    float m = -__builtin_inff();
    int has_nan = 0;
    for (int64_t j = lane; j < nbr; j += 64) {
      uint32_t v[32];
      load_block<false>(srow, j, v);
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        has_nan |= (v[k] & 0x7FFFFFFFu) > 0x7F800000u;
        m = fmaxf(m, __uint_as_float(v[k]));
      }
    }
    m = wave_max(m);
    if (wave_or(has_nan)) m = __builtin_nanf("");
    // pass 2: P = exp(s - m), then quantize each block of P
    for (int64_t j = lane; j < nbr; j += 64) {
      uint32_t v[32], c[32], o[W];
      float r[32];
      load_block<false>(srow, j, v);
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = __float_as_uint(exp_fixed(__uint_as_float(v[k]) - m));
      const uint32_t byte = quantize_regs<F>(v, c, r);
      pack32<W>(c, o);
      const int64_t b = row * nbr + j;
      store_codes<W>(codes, b, o);
      scales[b] = (uint8_t)byte;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline dim3 grid_for(int64_t work, int per_wg) {
  int64_t g = (work + per_wg - 1) / per_wg;
  if (g > 0x7FFFFFFF) g = 0x7FFFFFFF;
  if (g < 1) g = 1;
  return dim3((unsigned)g);
}

#define MXK_SWITCH_FMT(fmt, BODY)                 \
  switch (fmt) {                                  \
    case F_E2M3: { constexpr int FF = F_E2M3; BODY; } break; \
    case F_E3M2: { constexpr int FF = F_E3M2; BODY; } break; \
    case F_E2M1: { constexpr int FF = F_E2M1; BODY; } break; \
    case F_E4M3: { constexpr int FF = F_E4M3; BODY; } break; \
    case F_AXS6: { constexpr int FF = F_AXS6; BODY; } break; \
    default: return hipErrorInvalidValue;         \
  }

hipError_t launch_quantize(int fmt, bool bf16, const void* x, int64_t nb, void* codes,
                           uint8_t* scales, uint8_t* aux, hipStream_t st) {
  const dim3 grid = grid_for(nb, 256), block(256);
  MXK_SWITCH_FMT(fmt, {
    if (bf16) hipLaunchKernelGGL((quantize_lpb<FF, true>), grid, block, 0, st, x, nb, codes, scales, aux);
    else hipLaunchKernelGGL((quantize_lpb<FF, false>), grid, block, 0, st, x, nb, codes, scales, aux);
  });
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, bool bf16, const void* codes, const uint8_t* scales,
                             const uint8_t* aux, int64_t nb, void* y, hipStream_t st) {
  const dim3 grid = grid_for(nb, 256), block(256);
  MXK_SWITCH_FMT(fmt, {
    if (bf16) hipLaunchKernelGGL((dequantize_lpb<FF, true>), grid, block, 0, st, codes, scales, aux, nb, y);
    else hipLaunchKernelGGL((dequantize_lpb<FF, false>), grid, block, 0, st, codes, scales, aux, nb, y);
  });
  return hipGetLastError();
}

hipError_t launch_fake_quantize(int fmt, bool bf16, const void* x, int64_t nb, void* y,
                                hipStream_t st) {
  const dim3 grid = grid_for(nb, 256), block(256);
  MXK_SWITCH_FMT(fmt, {
    if (bf16) hipLaunchKernelGGL((fake_quantize_lpb<FF, true>), grid, block, 0, st, x, nb, y);
    else hipLaunchKernelGGL((fake_quantize_lpb<FF, false>), grid, block, 0, st, x, nb, y);
  });
  return hipGetLastError();
}

hipError_t launch_softmax_quantize(int fmt, const float* s, int64_t rows, int64_t cols,
                                   void* codes, uint8_t* scales, hipStream_t st) {
  const dim3 grid = grid_for(rows, 4), block(256);
  switch (fmt) {
    case F_E2M3: hipLaunchKernelGGL((softmax_quantize_rows<F_E2M3>), grid, block, 0, st, s, rows, cols, codes, scales); break;
    case F_E3M2: hipLaunchKernelGGL((softmax_quantize_rows<F_E3M2>), grid, block, 0, st, s, rows, cols, codes, scales); break;
    case F_E2M1: hipLaunchKernelGGL((softmax_quantize_rows<F_E2M1>), grid, block, 0, st, s, rows, cols, codes, scales); break;
    case F_E4M3: hipLaunchKernelGGL((softmax_quantize_rows<F_E4M3>), grid, block, 0, st, s, rows, cols, codes, scales); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mxk
