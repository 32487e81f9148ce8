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

// The floor of the exp-then-quantize prologue's byte mix on rows of 4096
// fp32 scores: the same grid (one wave per row, four per workgroup), the
// same loads (lanes 2i and 2i+1 read the two 64-byte halves of a block,
// the whole row before any store) and the same stores (8 code bytes per
// half block, the scale byte from the even lane), with the exp and the
// conversion replaced by folding the loaded words.
__global__ __launch_bounds__(256) void rows_floor(const uint4* __restrict__ s, int64_t rows,
                                                  uint2* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* src = s + row * 1024 + 4 * lane;  // 4096 floats = 1024 uint4
  uint4 keep[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) keep[g][j] = src[256 * g + j];
  uint32_t m = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) m ^= keep[g][j].x ^ keep[g][j].y ^ keep[g][j].z ^ keep[g][j].w;
  m ^= (uint32_t)__builtin_amdgcn_readfirstlane((int)m);  // a wave-wide step, like the row max
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t h = row * 256 + 64 * g + lane;
    const uint32_t w0 = keep[g][0].x ^ keep[g][1].y ^ keep[g][2].z ^ keep[g][3].w ^ m;
    const uint32_t w1 = keep[g][0].y ^ keep[g][1].z ^ keep[g][2].w ^ keep[g][3].x;
    const uint32_t w2 = keep[g][0].z ^ keep[g][1].w ^ keep[g][2].x ^ keep[g][3].y;
    const uint32_t w3 = keep[g][0].w ^ keep[g][1].x ^ keep[g][2].y ^ keep[g][3].z;
    codes[h] = make_uint2(w0 ^ w2, w1 ^ w3);
    if (!(lane & 1)) scales[h >> 1] = (uint8_t)(w0 >> 24);
  }
}

// s: [rows, 4096] fp32; codes: rows * 2048 bytes; scales: rows * 128 bytes
// (device memory, 16-byte aligned).  Other column counts: -1.
extern "C" int probe_rows_floor(const void* s, int64_t rows, int64_t cols, void* codes,
                                uint8_t* scales, void* stream) {
  if (cols != 4096 || rows < 1 || (rows + 3) / 4 > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(rows_floor, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(s), rows,
                     static_cast<uint2*>(codes), scales);
  return (int)hipGetLastError();
}
