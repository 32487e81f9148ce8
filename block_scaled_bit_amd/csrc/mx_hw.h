// mx_hw.h -- gfx950 scaled-conversion instructions wrapped per element
// format (device code only).
//
// The scale operand of every v_cvt_scalef32_* instruction is an fp32 whose
// exponent field is the E8M0 byte (byte << 23): the instruction divides by
// 2^(byte - 127) when encoding and multiplies by it when decoding.  The
// encodings round to nearest even and saturate for FP6 and FP4; the FP8
// encoding does not saturate, so a rounded magnitude of 0x7F (NaN) is mapped
// back to 0x7E (448), which is what clamp-then-round gives for every value a
// block can hold (|v| / X < 512).  The library's tests check each of these
// facts exhaustively against the CPU reference before the kernels rely on
// them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_formats.h"

namespace mxk {

typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x32_t __attribute__((ext_vector_type(32)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float scale_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// Largest |value| of 32 bf16 held as 16 dwords, as an fp32 bit pattern
// (bf16 pattern << 16): packed 16-bit unsigned max over the sign-cleared
// halves; NaN and inf patterns order above every finite one.
__device__ __forceinline__ uint32_t amax_bf16x32(const uint32_t (&d)[16]) {
  u16x2_t m = {0, 0};
#pragma unroll
  for (int k = 0; k < 16; ++k)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, d[k] & 0x7FFF7FFFu));
  const uint32_t lo = m[0], hi = m[1];
  return (hi > lo ? hi : lo) << 16;
}

// The same for 32 fp16: finite fp16 magnitudes also order as their bit
// patterns, with inf and NaN above them; the result is widened exactly to
// an fp32 pattern (inf and NaN stay non-finite).
__device__ __forceinline__ uint32_t amax_f16x32(const uint32_t (&d)[16]) {
  u16x2_t m = {0, 0};
#pragma unroll
  for (int k = 0; k < 16; ++k)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, d[k] & 0x7FFF7FFFu));
  const uint16_t h = m[1] > m[0] ? m[1] : m[0];
  return __float_as_uint((float)__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint32_t amax_f32x32(const uint32_t (&d)[32]) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 32; ++k) m = max(m, d[k] & 0x7FFFFFFFu);
  return m;
}

// FP8 E4M3: a rounded magnitude 0x7F in any byte becomes 0x7E.
__device__ __forceinline__ uint32_t e4m3_saturate4(uint32_t w) {
  const uint32_t t = w & 0x7F7F7F7Fu;
  const uint32_t nan_bytes = (t + 0x01010101u) & 0x80808080u;  // bytes whose magnitude is 0x7F
  return w - (nan_bytes >> 7);
}

// ---------------------------------------------------------------------------
// Encode one block of 32 values under scale operand sc into W code dwords.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void encode_bf16(const uint32_t (&d)[16], float sc, uint32_t (&o)[Fmt<F>::W]) {
  if constexpr (F == F_E2M3 || F == F_E3M2) {
    u32x16_t u;
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = d[k];
    const bf16x32_t v = __builtin_bit_cast(bf16x32_t, u);
    u32x6_t r;
    if constexpr (F == F_E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, sc);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(v, sc);
#pragma unroll
    for (int k = 0; k < 6; ++k) o[k] = r[k];
  } else if constexpr (F == F_E2M1) {
    // dword j holds elements 8j..8j+7: byte s from the bf16 pair d[4j+s]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, d[4 * j + 0]), sc, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, d[4 * j + 1]), sc, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, d[4 * j + 2]), sc, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, d[4 * j + 3]), sc, 3);
      o[j] = w;
    }
  } else {
    static_assert(F == F_E4M3, "hardware encode covers the MX formats");
    // dword j holds elements 4j..4j+3: low word from d[2j], high from d[2j+1]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s16x2_t w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w, __builtin_bit_cast(bf16x2_t, d[2 * j]), sc, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w, __builtin_bit_cast(bf16x2_t, d[2 * j + 1]), sc, true);
      o[j] = e4m3_saturate4(__builtin_bit_cast(uint32_t, w));
    }
  }
}

// The same from 32 fp16 held as 16 dwords (element 2k in the low half of
// dword k), with the fp16-source forms of the instructions.
template <int F>
__device__ __forceinline__ void encode_f16(const uint32_t (&d)[16], float sc, uint32_t (&o)[Fmt<F>::W]) {
  if constexpr (F == F_E2M3 || F == F_E3M2) {
    u32x16_t u;
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = d[k];
    const f16x32_t v = __builtin_bit_cast(f16x32_t, u);
    u32x6_t r;
    if constexpr (F == F_E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(v, sc);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_f16(v, sc);
#pragma unroll
    for (int k = 0; k < 6; ++k) o[k] = r[k];
  } else if constexpr (F == F_E2M1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(w, __builtin_bit_cast(f16x2_t, d[4 * j + 0]), sc, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(w, __builtin_bit_cast(f16x2_t, d[4 * j + 1]), sc, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(w, __builtin_bit_cast(f16x2_t, d[4 * j + 2]), sc, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(w, __builtin_bit_cast(f16x2_t, d[4 * j + 3]), sc, 3);
      o[j] = w;
    }
  } else {
    static_assert(F == F_E4M3, "hardware encode covers the MX formats");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s16x2_t w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, __builtin_bit_cast(f16x2_t, d[2 * j]), sc, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, __builtin_bit_cast(f16x2_t, d[2 * j + 1]), sc, true);
      o[j] = e4m3_saturate4(__builtin_bit_cast(uint32_t, w));
    }
  }
}

template <int F>
__device__ __forceinline__ void encode_f32(const uint32_t (&d)[32], float sc, uint32_t (&o)[Fmt<F>::W]) {
  if constexpr (F == F_E2M3 || F == F_E3M2) {
    // the instruction places a[k] at code 2k and b[k] at code 2k+1
    f32x16_t a, b;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      a[k] = __uint_as_float(d[2 * k]);
      b[k] = __uint_as_float(d[2 * k + 1]);
    }
    u32x6_t r;
    if constexpr (F == F_E2M3) r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, sc);
    else r = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, sc);
#pragma unroll
    for (int k = 0; k < 6; ++k) o[k] = r[k];
  } else if constexpr (F == F_E2M1) {
#define MXK_FP4_F32(w, j, s) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(d[8 * (j) + 2 * (s)]), \
                                           __uint_as_float(d[8 * (j) + 2 * (s) + 1]), sc, s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
      w = MXK_FP4_F32(w, j, 0);
      w = MXK_FP4_F32(w, j, 1);
      w = MXK_FP4_F32(w, j, 2);
      w = MXK_FP4_F32(w, j, 3);
      o[j] = w;
    }
#undef MXK_FP4_F32
  } else {
    static_assert(F == F_E4M3, "hardware encode covers the MX formats");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s16x2_t w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __uint_as_float(d[4 * j]), __uint_as_float(d[4 * j + 1]), sc, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __uint_as_float(d[4 * j + 2]), __uint_as_float(d[4 * j + 3]), sc, true);
      o[j] = e4m3_saturate4(__builtin_bit_cast(uint32_t, w));
    }
  }
}

// ---------------------------------------------------------------------------
// Encode one half block (values 16h..16h+15 of a block, as fp32 patterns)
// under sc into the W/2 code dwords that hold exactly those values (the
// packed layouts above put the first 16 codes in the first W/2 dwords).
// FP6: the 32-wide instruction with its last 16 inputs zero, whose codes
// land in the dwords that are dropped.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void encode_f32_half(const uint32_t (&d)[16], float sc,
                                                uint32_t (&o)[Fmt<F>::W / 2]) {
  if constexpr (F == F_E2M3 || F == F_E3M2) {
    f32x16_t a, b;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      a[k] = k < 8 ? __uint_as_float(d[2 * k]) : 0.0f;
      b[k] = k < 8 ? __uint_as_float(d[2 * k + 1]) : 0.0f;
    }
    u32x6_t r;
    if constexpr (F == F_E2M3) r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, sc);
    else r = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, sc);
#pragma unroll
    for (int k = 0; k < 3; ++k) o[k] = r[k];
  } else if constexpr (F == F_E2M1) {
#define MXK_FP4_F32(w, j, s) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(d[8 * (j) + 2 * (s)]), \
                                           __uint_as_float(d[8 * (j) + 2 * (s) + 1]), sc, s)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w = 0;
      w = MXK_FP4_F32(w, j, 0);
      w = MXK_FP4_F32(w, j, 1);
      w = MXK_FP4_F32(w, j, 2);
      w = MXK_FP4_F32(w, j, 3);
      o[j] = w;
    }
#undef MXK_FP4_F32
  } else {
    static_assert(F == F_E4M3, "hardware encode covers the MX formats");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s16x2_t w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __uint_as_float(d[4 * j]), __uint_as_float(d[4 * j + 1]), sc, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __uint_as_float(d[4 * j + 2]), __uint_as_float(d[4 * j + 3]), sc, true);
      o[j] = e4m3_saturate4(__builtin_bit_cast(uint32_t, w));
    }
  }
}

// ---------------------------------------------------------------------------
// Decode one block of W code dwords under sc: 32 bf16 as 16 dwords, or 32
// fp32 bit patterns.  NaN results (E4M3 NaN codes) are left as the
// instruction produces them; the caller canonicalizes.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void decode_bf16(const uint32_t (&o)[Fmt<F>::W], float sc, uint32_t (&d)[16]) {
  if constexpr (F == F_E2M3 || F == F_E3M2) {
    u32x6_t c;
#pragma unroll
    for (int k = 0; k < 6; ++k) c[k] = o[k];
    bf16x32_t r;
    if constexpr (F == F_E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(c, sc);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(c, sc);
    const u32x16_t u = __builtin_bit_cast(u32x16_t, r);
#pragma unroll
    for (int k = 0; k < 16; ++k) d[k] = u[k];
  } else if constexpr (F == F_E2M1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[4 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(o[j], sc, 0));
      d[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(o[j], sc, 1));
      d[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(o[j], sc, 2));
      d[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(o[j], sc, 3));
    }
  } else {
    static_assert(F == F_E4M3, "hardware decode covers the MX formats");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      d[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(o[j], sc, false));
      d[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(o[j], sc, true));
    }
  }
}

template <int F>
__device__ __forceinline__ void decode_f32(const uint32_t (&o)[Fmt<F>::W], float sc, uint32_t (&d)[32]) {
  if constexpr (F == F_E2M3 || F == F_E3M2) {
    u32x6_t c;
#pragma unroll
    for (int k = 0; k < 6; ++k) c[k] = o[k];
    f32x32_t r;
    if constexpr (F == F_E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, sc);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(c, sc);
#pragma unroll
    for (int k = 0; k < 32; ++k) d[k] = __float_as_uint(r[k]);
  } else if constexpr (F == F_E2M1) {
#define MXK_F32_FP4(j, s)                                                      \
  do {                                                                         \
    const f32x2_t r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o[j], sc, s);   \
    d[8 * (j) + 2 * (s)] = __float_as_uint(r[0]);                              \
    d[8 * (j) + 2 * (s) + 1] = __float_as_uint(r[1]);                          \
  } while (0)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      MXK_F32_FP4(j, 0);
      MXK_F32_FP4(j, 1);
      MXK_F32_FP4(j, 2);
      MXK_F32_FP4(j, 3);
    }
#undef MXK_F32_FP4
  } else {
    static_assert(F == F_E4M3, "hardware decode covers the MX formats");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(o[j], sc, false);
      const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(o[j], sc, true);
      d[4 * j] = __float_as_uint(lo[0]);
      d[4 * j + 1] = __float_as_uint(lo[1]);
      d[4 * j + 2] = __float_as_uint(hi[0]);
      d[4 * j + 3] = __float_as_uint(hi[1]);
    }
  }
}

// Does any E4M3 code of the block have the NaN magnitude 0x7F?
__device__ __forceinline__ bool e4m3_has_nan_code(const uint32_t (&o)[8]) {
  uint32_t any = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t t = o[j] & 0x7F7F7F7Fu;
    any |= (t + 0x01010101u) & 0x80808080u;
  }
  return any != 0;
}

}  // namespace mxk
