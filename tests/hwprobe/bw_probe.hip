// bw_probe.hip -- the HBM ceiling of the bf16 -> FP6 quantizer's byte mix.
//
// A copy kernel with the quantizer's layout, grid and memory instructions
// (one lane per 32-value block: four 16-byte loads of its 64 bf16 bytes,
// three 8-byte stores of 24 "code" bytes, one scale byte) and no
// arithmetic beyond folding every input word into the outputs, so that the
// compiler keeps every load.  The benchmark times it beside the quantizer
// on the same buffers; it is measurement infrastructure, not part of the
// library.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ __launch_bounds__(256) void mix_copy(const uint4* __restrict__ x, int64_t nb,
                                                uint2* __restrict__ codes,
                                                uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    const uint4 q0 = x[4 * b], q1 = x[4 * b + 1], q2 = x[4 * b + 2], q3 = x[4 * b + 3];
    const uint32_t o0 = q0.x ^ q2.z, o1 = q0.y ^ q2.w, o2 = q0.z ^ q3.x, o3 = q0.w ^ q3.y;
    const uint32_t o4 = q1.x ^ q1.z ^ q3.z, o5 = q1.y ^ q1.w ^ q3.w ^ q2.x ^ q2.y;
    codes[3 * b] = make_uint2(o0, o1);
    codes[3 * b + 1] = make_uint2(o2, o3);
    codes[3 * b + 2] = make_uint2(o4, o5);
    scales[b] = (uint8_t)(o0 ^ o5);
  }
}

// x: nb blocks of 64 bytes; codes: nb * 24 bytes; scales: nb bytes (all
// device memory, 16-byte aligned).  Returns hipGetLastError().
extern "C" int probe_mix_copy(const void* x, int64_t nb, void* codes, uint8_t* scales,
                              void* stream) {
  int64_t g = (nb + 255) / 256;
  if (g > 0x7FFFFFFF) g = 0x7FFFFFFF;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(mix_copy, dim3((unsigned)g), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(x), nb, static_cast<uint2*>(codes), scales);
  return (int)hipGetLastError();
}
