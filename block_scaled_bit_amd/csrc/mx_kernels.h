// mx_kernels.h -- internal launchers of the gfx950 kernels (not part of the
// C ABI).  Each enqueues one kernel on `st` and returns hipGetLastError().
// Formats: 0 E2M3, 1 E3M2, 2 E2M1, 3 E4M3, 4 AXS-6.  nb = number of 32-value
// blocks.  Arguments are validated by the C-ABI layer before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

// Generic eXmY format parameters (prepared on the host): m mantissa bits;
// emin = exponent of the smallest normal (m for integer formats); emax =
// floor(log2 of the largest magnitude); bias = 1 - emin; maxf = the largest
// magnitude (e8m0: half of it, 2^127); dec_bits, dec_sub as below.
struct ExmyParams {
  int m;
  int emin;
  int emax;
  int bias;
  float maxf;
  // decoding constants: the fp32 exponent-field offset (127 - bias) << 23
  // and -2^(1 - bias)
  uint32_t dec_bits;
  float dec_sub;
};

// dt: the tensor element type, as the C ABI's mx_dtype (0 bf16, 1 fp32,
// 2 fp16).
hipError_t launch_quantize(int fmt, int dt, const void* x, int64_t nb, void* codes,
                           uint8_t* scales, uint8_t* aux, hipStream_t st);

// Up to kBatchMax tensors of one MX hardware format (E2M3, E3M2, E2M1,
// E4M3) quantized by one launch, passed by value as the kernel argument:
// tensor i has nb[i] > 0 blocks and owns workgroups [wg_start[i],
// wg_start[i + 1]) of 256 blocks each; wg_start[0] = 0 and wg_start[n] is
// the grid size.
constexpr int kBatchMax = 16;
struct QuantBatch {
  int n;
  uint32_t wg_start[kBatchMax + 1];
  int64_t nb[kBatchMax];
  const void* x[kBatchMax];
  void* codes[kBatchMax];
  uint8_t* scales[kBatchMax];
};
hipError_t launch_quantize_batch(int fmt, int dt, const QuantBatch& a, hipStream_t st);
hipError_t launch_dequantize(int fmt, int dt, const void* codes, const uint8_t* scales,
                             const uint8_t* aux, int64_t nb, void* y, hipStream_t st);
hipError_t launch_fake_quantize(int fmt, int dt, const void* x, int64_t nb, void* y,
                                hipStream_t st);
// op 0: quantize (in = x, out = codes, scales_out); op 1: dequantize (in =
// codes, scales_in, out = y); op 2: fake-quantize (in = x, out = y).
hipError_t launch_exmy(int op, int width, const ExmyParams& p, int dt, const void* in,
                       const uint8_t* scales_in, int64_t nb, void* out, uint8_t* scales_out,
                       hipStream_t st);
hipError_t launch_softmax_quantize(int fmt, const float* s, int64_t rows, int64_t cols,
                                   void* codes, uint8_t* scales, hipStream_t st);
// Attention forward with E2M1 probabilities (efq: the exp-free EFQ reading
// instead of exp-then-quantize); head dimension 128, v_fmt one of E2M3,
// E3M2, E2M1, E4M3; row_max, row_sum, p_codes, p_scales may be NULL
// (p_codes and p_scales together).
hipError_t launch_attention(int v_fmt, bool efq, bool out_bf16, const void* q, const void* k,
                            const void* v_codes, const uint8_t* v_scales, int heads, int lq,
                            int lk, float scale, void* o, float* row_max, float* row_sum,
                            void* p_codes, uint8_t* p_scales, hipStream_t st);

}  // namespace mxk
