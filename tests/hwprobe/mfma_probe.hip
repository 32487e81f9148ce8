// mfma_probe.hip -- test-only kernels that run one gfx950 matrix
// instruction (or one lane permutation) on per-lane register contents given
// by the host, so the tests can check the operand and result layouts the
// attention kernel assumes.  Every kernel runs as one wave of 64 lanes and
// touches lanes 0..63 of its buffers only.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// D = A * B + C with block scales; a, b: 8 dwords per lane; sa, sb: one
// E8M0 byte per lane (byte 0 of the scale operand); d: 16 floats per lane,
// read as C and overwritten with D.  C comes from memory on purpose: with a
// constant zero accumulator this compiler may place the result over the A
// and B registers, which the instruction still reads for fp8 A operands.
template <int FA, int FB>
__global__ void k_mfma_scale_32x32x64(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                                      const uint32_t* sb, float* d) {
  const int l = threadIdx.x;
  i32x8 ra, rb;
  for (int i = 0; i < 8; ++i) { ra[i] = (int)a[8 * l + i]; rb[i] = (int)b[8 * l + i]; }
  f32x16 c;
  for (int i = 0; i < 16; ++i) c[i] = d[16 * l + i];
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ra, rb, c, FA, FB, 0, (int)sa[l], 0,
                                                      (int)sb[l]);
  for (int i = 0; i < 16; ++i) d[16 * l + i] = c[i];
}

// D = A * B + C for 32x32x16 bf16; a, b: 4 dwords (8 bf16) per lane; d
// as above
__global__ void k_mfma_bf16_32x32x16(const uint32_t* a, const uint32_t* b, float* d) {
  const int l = threadIdx.x;
  u32x4 ua, ub;
  for (int i = 0; i < 4; ++i) { ua[i] = a[4 * l + i]; ub[i] = b[4 * l + i]; }
  f32x16 c;
  for (int i = 0; i < 16; ++i) c[i] = d[16 * l + i];
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ua),
                                              __builtin_bit_cast(bf16x8, ub), c, 0, 0, 0);
  for (int i = 0; i < 16; ++i) d[16 * l + i] = c[i];
}

// v_permlane32_swap on (x, y); results back into x and y
__global__ void k_permlane32_swap(uint32_t* x, uint32_t* y) {
  const int l = threadIdx.x;
  auto r = __builtin_amdgcn_permlane32_swap(x[l], y[l], false, false);
  x[l] = r[0];
  y[l] = r[1];
}

#define ONE_WAVE dim3(1), dim3(64), 0, (hipStream_t)0
extern "C" {
// fa, fb: 0 E4M3, 2 E2M3, 3 E3M2, 4 E2M1 (the instruction's format codes)
int probe_mfma_scale(int fa, int fb, const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                     const uint32_t* sb, float* d) {
#define CASE(A, B)                                                                    \
  if (fa == A && fb == B) {                                                           \
    hipLaunchKernelGGL((k_mfma_scale_32x32x64<A, B>), ONE_WAVE, a, b, sa, sb, d);      \
    return (int)hipDeviceSynchronize();                                               \
  }
  CASE(0, 0) CASE(0, 4) CASE(2, 4) CASE(3, 4) CASE(4, 4) CASE(4, 0)
#undef CASE
  return -1;
}
int probe_mfma_bf16(const uint32_t* a, const uint32_t* b, float* d) {
  hipLaunchKernelGGL(k_mfma_bf16_32x32x16, ONE_WAVE, a, b, d);
  return (int)hipDeviceSynchronize();
}
int probe_permlane32_swap(uint32_t* x, uint32_t* y) {
  hipLaunchKernelGGL(k_permlane32_swap, ONE_WAVE, x, y);
  return (int)hipDeviceSynchronize();
}
}
