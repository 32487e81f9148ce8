// cvt_probe.hip -- test-only kernels that run gfx950's scaled conversion
// instructions on given inputs, so the tests can compare them exhaustively
// with the CPU oracle before the library relies on any of them.  Each lane
// converts one input group with one scale byte (placed in the exponent
// field of the fp32 scale operand).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x32 __attribute__((ext_vector_type(32)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef short shortx2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float scale_of(uint32_t byte) { return __uint_as_float(byte << 23); }

// 32 bf16 (16 dwords) -> 32 fp6 codes (6 dwords); kind 0: E2M3, 1: E3M2
__global__ void k_q_fp6_bf16(int kind, const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u32x16 u;
  for (int k = 0; k < 16; ++k) u[k] = in[16 * i + k];
  bf16x32 v = __builtin_bit_cast(bf16x32, u);
  u32x6 r = kind == 0 ? __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, scale_of(sb[i]))
                      : __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(v, scale_of(sb[i]));
  for (int k = 0; k < 6; ++k) out[6 * i + k] = r[k];
}

// 32 fp16 (16 dwords) -> 32 fp6 codes (6 dwords); kind 0: E2M3, 1: E3M2
__global__ void k_q_fp6_f16(int kind, const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u32x16 u;
  for (int k = 0; k < 16; ++k) u[k] = in[16 * i + k];
  f16x32 v = __builtin_bit_cast(f16x32, u);
  u32x6 r = kind == 0 ? __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(v, scale_of(sb[i]))
                      : __builtin_amdgcn_cvt_scalef32_pk32_bf6_f16(v, scale_of(sb[i]));
  for (int k = 0; k < 6; ++k) out[6 * i + k] = r[k];
}

// 32 fp32 (two groups of 16) -> 32 fp6 codes
__global__ void k_q_fp6_f32(int kind, const float* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  // the instruction interleaves its operands: code 2k comes from a[k] and
  // code 2k+1 from b[k]
  f32x16 a, b;
  for (int k = 0; k < 16; ++k) { a[k] = in[32 * i + 2 * k]; b[k] = in[32 * i + 2 * k + 1]; }
  u32x6 r = kind == 0 ? __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, scale_of(sb[i]))
                      : __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, scale_of(sb[i]));
  for (int k = 0; k < 6; ++k) out[6 * i + k] = r[k];
}

// 2 bf16 (one dword) -> 2 E4M3 codes (low 16 bits of the result)
__global__ void k_q_fp8_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  bf16x2 v = __builtin_bit_cast(bf16x2, in[i]);
  shortx2 old = {0, 0};
  shortx2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(old, v, scale_of(sb[i]), false);
  out[i] = __builtin_bit_cast(uint32_t, r);
}

// 2 fp16 (one dword) -> 2 E4M3 codes (low 16 bits of the result)
__global__ void k_q_fp8_f16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  f16x2 v = __builtin_bit_cast(f16x2, in[i]);
  shortx2 old = {0, 0};
  shortx2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(old, v, scale_of(sb[i]), false);
  out[i] = __builtin_bit_cast(uint32_t, r);
}

// 2 fp32 -> 2 E4M3 codes
__global__ void k_q_fp8_f32(const float* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  shortx2 old = {0, 0};
  shortx2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, in[2 * i], in[2 * i + 1], scale_of(sb[i]), false);
  out[i] = __builtin_bit_cast(uint32_t, r);
}

// 2 bf16 -> 2 E2M1 codes (low byte)
__global__ void k_q_fp4_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  bf16x2 v = __builtin_bit_cast(bf16x2, in[i]);
  out[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, v, scale_of(sb[i]), 0);
}

// 2 fp16 -> 2 E2M1 codes (low byte)
__global__ void k_q_fp4_f16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  f16x2 v = __builtin_bit_cast(f16x2, in[i]);
  out[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(0u, v, scale_of(sb[i]), 0);
}

// 2 fp32 -> 2 E2M1 codes (low byte)
__global__ void k_q_fp4_f32(const float* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, in[2 * i], in[2 * i + 1], scale_of(sb[i]), 0);
}

// 32 fp6 codes (6 dwords) -> 32 bf16 (16 dwords) / 32 fp32
__global__ void k_dq_fp6_bf16(int kind, const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u32x6 c;
  for (int k = 0; k < 6; ++k) c[k] = in[6 * i + k];
  bf16x32 r = kind == 0 ? __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(c, scale_of(sb[i]))
                        : __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(c, scale_of(sb[i]));
  u32x16 u = __builtin_bit_cast(u32x16, r);
  for (int k = 0; k < 16; ++k) out[16 * i + k] = u[k];
}

__global__ void k_dq_fp6_f32(int kind, const uint32_t* in, const uint8_t* sb, float* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u32x6 c;
  for (int k = 0; k < 6; ++k) c[k] = in[6 * i + k];
  f32x32 r = kind == 0 ? __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, scale_of(sb[i]))
                       : __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(c, scale_of(sb[i]));
  for (int k = 0; k < 32; ++k) out[32 * i + k] = r[k];
}

// low 2 codes of a dword: E4M3 -> 2 bf16 ; E2M1 (low byte) -> 2 bf16
__global__ void k_dq_fp8_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in[i], scale_of(sb[i]), false);
  out[i] = __builtin_bit_cast(uint32_t, r);
}

__global__ void k_dq_fp4_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(in[i], scale_of(sb[i]), 0);
  out[i] = __builtin_bit_cast(uint32_t, r);
}


// E2M1 / E4M3 codes (low 2 of a dword) -> 2 fp32
__global__ void k_dq_fp4_f32(const uint32_t* in, const uint8_t* sb, float* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float2v r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(in[i], scale_of(sb[i]), 0);
  out[2 * i] = r[0];
  out[2 * i + 1] = r[1];
}
__global__ void k_dq_fp8_f32(const uint32_t* in, const uint8_t* sb, float* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float2v r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(in[i], scale_of(sb[i]), false);
  out[2 * i] = r[0];
  out[2 * i + 1] = r[1];
}

#define GRID(n) dim3(((n) + 255) / 256), dim3(256), 0, (hipStream_t)0
extern "C" {
int probe_q_fp6_bf16(int kind, const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp6_bf16, GRID(n), kind, in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp6_f32(int kind, const float* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp6_f32, GRID(n), kind, in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp6_f16(int kind, const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp6_f16, GRID(n), kind, in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp8_f16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp8_f16, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp4_f16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp4_f16, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp8_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp8_bf16, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp8_f32(const float* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp8_f32, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp4_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp4_bf16, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_q_fp4_f32(const float* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_q_fp4_f32, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_dq_fp6_bf16(int kind, const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_dq_fp6_bf16, GRID(n), kind, in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_dq_fp6_f32(int kind, const uint32_t* in, const uint8_t* sb, float* out, int n) {
  hipLaunchKernelGGL(k_dq_fp6_f32, GRID(n), kind, in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_dq_fp8_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_dq_fp8_bf16, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_dq_fp4_f32(const uint32_t* in, const uint8_t* sb, float* out, int n) {
  hipLaunchKernelGGL(k_dq_fp4_f32, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_dq_fp8_f32(const uint32_t* in, const uint8_t* sb, float* out, int n) {
  hipLaunchKernelGGL(k_dq_fp8_f32, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
int probe_dq_fp4_bf16(const uint32_t* in, const uint8_t* sb, uint32_t* out, int n) {
  hipLaunchKernelGGL(k_dq_fp4_bf16, GRID(n), in, sb, out, n); return (int)hipDeviceSynchronize(); }
}
