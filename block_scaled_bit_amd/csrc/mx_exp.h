// mx_exp.h -- the fixed fp32 exp of the stand-alone exp-then-quantize
// probabilities (device code only).
//
// Cody-Waite reduction (Cody and Waite, "Software Manual for the Elementary
// Functions", 1980) with ln2 split into a 16-bit head and a tail, a degree-7
// Taylor polynomial by Horner's rule with fused multiply-adds, and one
// scaling by 2^n with a single rounding.  Constants: log2(e), ln2 and 1/k!
// rounded to fp32; head = ln2's fp32 significand cut to 16 bits, tail =
// fp32(ln2 - head).  The sequence is a contract: the CPU reference runs the
// same operations, so probabilities agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>

namespace mxk {

// exp(d) for d <= 0 (shifted scores) and d = -inf (-> 0).  The reduction
// runs on max(d, -104): from there the product below already rounds to +0,
// which is the exact result for every d < -104 too.  The caller guarantees
// d is not NaN.
__device__ __forceinline__ float exp_ref_nonpos(float d) {
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.62e400p-1f;
  const float kLn2Lo = 0x1.7f7d1cp-20f;
  const float k2 = 0x1.000000p-1f, k3 = 0x1.555556p-3f, k4 = 0x1.555556p-5f,
              k5 = 0x1.111112p-7f, k6 = 0x1.6c16c2p-10f, k7 = 0x1.a01a02p-13f;
  const float dc = __builtin_fmaxf(d, -104.0f);
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
  // p * 2^n with one rounding (n in [-150, 0]; subnormal results rounded to
  // nearest even), the same value as exact power-of-two pre-scaling
  return __builtin_ldexpf(p, (int)nf);
}

}  // namespace mxk
