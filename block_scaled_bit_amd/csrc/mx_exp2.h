// mx_exp2.h -- the fixed fp32 2^u of the attention forward's probabilities
// (device code only).
//
// The attention forward folds log2(e) into its score scale, so its
// probabilities are 2^u of shifted scores u <= 0 already in powers of two.
// The sequence: n = rint(u), f = u - n (exact, |f| <= 1/2), a degree-5
// polynomial 1 + c1 f + ... + c5 f^5 in f by Horner's rule with fused
// multiply-adds, and one scaling by 2^n with a single rounding.  The
// coefficients minimize the largest relative error over [-1/2, 1/2] with
// the constant term held at exactly 1 (a linear program on a dense grid),
// each then moved by a few fp32 ulps to the values whose fp32 evaluation
// errs least: the result is within 2.1 ulp of 2^u, and exact for integer u
// down to -149.  The sequence is a contract: the CPU reference runs the same
// operations, so probabilities agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>

namespace mxk {

__device__ __forceinline__ float exp2_poly(float f) {
  const float c1 = 0x1.62e42ap-1f, c2 = 0x1.ebf994p-3f, c3 = 0x1.c6b5acp-5f, c4 = 0x1.3cf68ap-7f,
              c5 = 0x1.5c54b4p-10f;
  float p = c5;
  p = __builtin_fmaf(p, f, c4);
  p = __builtin_fmaf(p, f, c3);
  p = __builtin_fmaf(p, f, c2);
  p = __builtin_fmaf(p, f, c1);
  p = __builtin_fmaf(p, f, 1.0f);
  return p;
}

// float -> int32 as v_cvt_i32_f32 defines it for every input (toward zero,
// saturating at the int32 limits, NaN -> 0); a C conversion of an
// out-of-range value would be undefined.
__device__ __forceinline__ int cvt_i32_sat(float x) {
  int r;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// 2^u for u <= 0 and u = -inf (-> 0).  The reduction runs on max(u, -151):
// from there 2^n p already rounds to +0, the exact result for every
// u < -151 too.  kNaN: a NaN u gives NaN (the clamp is then a comparison,
// one more instruction); otherwise the caller guarantees u is not NaN.
template <bool kNaN = false>
__device__ __forceinline__ float exp2_ref_nonpos(float u) {
  const float uc = kNaN ? (u < -151.0f ? -151.0f : u) : __builtin_fmaxf(u, -151.0f);
  const float nf = __builtin_rintf(uc);
  return __builtin_ldexpf(exp2_poly(uc - nf), (int)nf);
}

// The same sequence without the clamp, for callers that check the results.
// For every finite u <= 0 it equals exp2_ref_nonpos(u): below -151, n <=
// -151 and p < 1.5 put p 2^n under 2^-150, which rounds to +0 (for
// |u| >= 2^23, u is an integer, f = 0, p = 1 and n saturates); u = -inf
// gives f = -inf - (-inf) = NaN and so NaN, which the caller detects and
// recomputes with the clamp.
__device__ __forceinline__ float exp2_ref_nonpos_unclamped(float u) {
  const float nf = __builtin_rintf(u);
  return __builtin_ldexpf(exp2_poly(u - nf), cvt_i32_sat(nf));
}

}  // namespace mxk
