// mx_formats.h -- element-format traits and per-value device arithmetic for
// the gfx950 kernels (device code only; shared by the kernel sources).
//
// Formats ("Online MXFP6" page: OCP MXFP6 E2M3 / E3M2 with an E8M0 scale per
// 32 values; "EFQ-Softmax" explainer, "Jargon": E2M1; "AXS-6" page,
// "Overview": E4M3 layout and the AXS-6 sign + 5-bit mantissa block).
// Exponent biases and ranges are those of the OCP MX formats the MXFP6 page
// names.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

enum { F_E2M3 = 0, F_E3M2 = 1, F_E2M1 = 2, F_E4M3 = 3, F_AXS6 = 4 };

template <int F> struct Fmt;
// W: code bits; M: mantissa bits; BIAS; EMIN: exponent of the smallest
// normal; EMAX: floor(log2 of the largest finite value); MAXF: largest
// finite magnitude; NAN_MAG: magnitude code meaning NaN (or -1).
template <> struct Fmt<F_E2M3> {
  static constexpr int W = 6, M = 3, BIAS = 1, EMIN = 0, EMAX = 2, NAN_MAG = -1;
  static constexpr bool FIXED = false;
  static constexpr float MAXF = 7.5f;
};
template <> struct Fmt<F_E3M2> {
  static constexpr int W = 6, M = 2, BIAS = 3, EMIN = -2, EMAX = 4, NAN_MAG = -1;
  static constexpr bool FIXED = false;
  static constexpr float MAXF = 28.0f;
};
template <> struct Fmt<F_E2M1> {
  static constexpr int W = 4, M = 1, BIAS = 1, EMIN = 0, EMAX = 2, NAN_MAG = -1;
  static constexpr bool FIXED = false;
  static constexpr float MAXF = 6.0f;
};
template <> struct Fmt<F_E4M3> {
  static constexpr int W = 8, M = 3, BIAS = 7, EMIN = -6, EMAX = 8, NAN_MAG = 0x7F;
  static constexpr bool FIXED = false;
  static constexpr float MAXF = 448.0f;
};
// AXS-6: magnitude m (5 bits) means m/16 under the shared exponent, so the
// largest value 31/16 sits in binade 0.
template <> struct Fmt<F_AXS6> {
  static constexpr int W = 6, M = 4, BIAS = 0, EMIN = 0, EMAX = 0, NAN_MAG = -1;
  static constexpr bool FIXED = true;
  static constexpr float MAXF = 31.0f / 16.0f;
};

// Bytes of one packed 32-value block: 32 codes of W bits = W dwords.
template <int F> constexpr int bytes_per_block() { return Fmt<F>::W * 4; }

// ---------------------------------------------------------------------------
// Scale: from the largest |value| of a block, given as the fp32 bit pattern of
// that magnitude (a bf16 pattern shifted left by 16 is the same number).
// Patterns >= 0x7F800000 are infinities or NaNs: the block gets byte 0xFF.
// Otherwise byte = clamp(floor(log2 amax) - EMAX + 127, 0, 254), 0 for amax 0.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 0xFFu;
  if (amax_bits == 0u) return 0u;
  int field = (int)(amax_bits >> 23);
  // floor(log2): the exponent field for normals; the leading bit position
  // of the significand for subnormals (value = bits * 2^-149)
  int e = field ? field - 127 : (31 - __builtin_clz(amax_bits)) - 149;
  int b = e - Fmt<F>::EMAX + 127;
  b = b < 0 ? 0 : b;
  b = b > 254 ? 254 : b;
  return (uint32_t)b;
}

// ---------------------------------------------------------------------------
// AXS-6 in software (there is no hardware AXS-6 format).  The kernels round
// m = rint(|v| 2^(131 - byte)) (16 |v| / X exactly: a value small enough to
// lose bits in that power-of-two scaling rounds to 0 either way) to nearest
// even and clamp it to 31; decoding is the exact m 2^(byte - 131).
// ---------------------------------------------------------------------------
// Unscaled AXS-6 value m/16 times 2^scale_exp (exact in fp32).
template <int F>
__device__ __forceinline__ float decode_mag(uint32_t mag, int scale_exp) {
  static_assert(Fmt<F>::FIXED, "software decoding is used for AXS-6 only");
  return __builtin_ldexpf((float)mag, scale_exp - 4);
}

// fp32 -> bf16 bit pattern, round to nearest even; NaN -> canonical.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Bit packing: 32 codes of W bits -> W dwords, little-endian bit stream
// (code k at stream bits [k*W, k*W+W)).
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ void pack32(const uint32_t (&c)[32], uint32_t (&o)[W]) {
#pragma unroll
  for (int j = 0; j < W; ++j) o[j] = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int bit = k * W, j = bit >> 5, s = bit & 31;
    o[j] |= c[k] << s;
    if (s + W > 32) o[j + 1] |= c[k] >> (32 - s);
  }
}

template <int W>
__device__ __forceinline__ uint32_t unpack1(const uint32_t (&o)[W], int k) {
  const int bit = k * W, j = bit >> 5, s = bit & 31;
  uint32_t v = o[j] >> s;
  if (s + W > 32) v |= o[j + 1] << (32 - s);
  return v & ((1u << W) - 1u);
}

}  // namespace mxk
