// exp_probe.hip -- test-only kernels that apply the library's fixed
// exponentials (block_scaled_bit_amd/csrc/mx_exp.h, mx_exp2.h) element by
// element, so the tests can compare every result with the CPU reference
// bit for bit, independently of any quantization around them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_exp.h"
#include "mx_exp2.h"

namespace {

// form: 0 exp_ref_nonpos (base e, clamped); 1 exp2_ref_nonpos (clamped);
// 2 exp2_ref_nonpos<true> (NaN-preserving); 3 exp2_ref_nonpos_unclamped
__global__ void k_exp(int form, const float* __restrict__ in, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = in[i];
  float r;
  if (form == 0) r = mxk::exp_ref_nonpos(v);
  else if (form == 1) r = mxk::exp2_ref_nonpos(v);
  else if (form == 2) r = mxk::exp2_ref_nonpos<true>(v);
  else r = mxk::exp2_ref_nonpos_unclamped(v);
  out[i] = r;
}

}  // namespace

extern "C" int probe_exp(int form, const float* in, float* out, int64_t n) {
  if (n <= 0) return 0;
  if (form < 0 || form > 3) return -1;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(k_exp, dim3((unsigned)blocks), dim3(256), 0, 0, form, in, out, n);
  return (int)hipDeviceSynchronize();
}
