// mx_api.cpp -- the C ABI declared in include/mx.h: host-side validation and
// dispatch to the gfx950 kernels.  Nothing here allocates or keeps state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "mx.h"
#include "mx_kernels.h"

namespace {

constexpr int kBytesPerBlock[5] = {24, 24, 16, 32, 24};

bool is_exmy(int f) { return (f & ~0xFF) == 0x100; }
int exmy_e(int f) { return (f >> 4) & 0xF; }
int exmy_m(int f) { return f & 0xF; }
int exmy_width(int f) { return 1 + exmy_e(f) + exmy_m(f); }

bool fmt_ok(int f) {
  if (f >= MX_FP6_E2M3 && f <= MX_AXS6) return true;
  return is_exmy(f) && exmy_width(f) >= 3 && exmy_width(f) <= 9;
}

int bytes_per_block(int f) { return is_exmy(f) ? 4 * exmy_width(f) : kBytesPerBlock[f]; }

// The generic format's parameters: sign-magnitude, bias 2^(e-1) - 1 with
// subnormals and no special codes; e = 0 is an integer magnitude.
mxk::ExmyParams exmy_params(int f) {
  const int e = exmy_e(f), m = exmy_m(f);
  mxk::ExmyParams p;
  p.m = m;
  if (e >= 1) {
    const int bias = (1 << (e - 1)) - 1;
    p.emin = 1 - bias;
    p.emax = ((1 << e) - 1) - bias;
    // e8m0's largest magnitude, 2^128, is beyond fp32: its kernels clamp
    // half the scaled magnitude, at 2^127
    p.maxf = e == 8 ? ldexpf(1.0f, 127) : ldexpf(2.0f - ldexpf(1.0f, -m), p.emax);
  } else {
    p.emin = m;
    p.emax = m - 1;
    p.maxf = ldexpf(1.0f, m) - 1.0f;
  }
  p.bias = 1 - p.emin;
  p.dec_bits = (uint32_t)(127 - p.bias) << 23;
  p.dec_sub = -ldexpf(1.0f, 1 - p.bias);
  return p;
}
bool dtype_ok(int d) { return d == MX_BF16 || d == MX_FP32 || d == MX_FP16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common shape / format checks.  Sets *nothing = true for an empty tensor.
mx_status check_common(int fmt, int block, int64_t rows, int64_t cols, bool* nothing) {
  if (!fmt_ok(fmt)) return MX_ERR_UNSUPPORTED;
  if (block != MX_BLOCK) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  if (cols % MX_BLOCK != 0) return MX_ERR_SHAPE;
  // the element count must fit the byte offsets the kernels form
  if (rows > 0 && cols > 0 && rows > (INT64_MAX / 8) / cols) return MX_ERR_SHAPE;
  *nothing = (rows == 0 || cols == 0);
  return MX_OK;
}

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_DEVICE; }

// Test hook: with MX_TEST_FAIL_LAUNCH=1 in the environment (read once per
// process), every call that passes its argument checks returns
// MX_ERR_DEVICE instead of launching, so a caller's handling of device
// errors can be exercised on a machine without a GPU.
bool forced_launch_failure() {
  static const bool fail = [] {
    const char* e = getenv("MX_TEST_FAIL_LAUNCH");
    return e != nullptr && e[0] == '1' && e[1] == '\0';
  }();
  return fail;
}

}  // namespace

extern "C" {

int mx_abi_version(void) { return MX_ABI_VERSION; }

const char* mx_status_str(mx_status status) {
  switch ((int)status) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "bad shape: rows/cols must be >= 0 and cols a multiple of 32";
    case MX_ERR_ALIGN: return "x, y and codes must be 16-byte aligned";
    case MX_ERR_UNSUPPORTED: return "unsupported format, dtype or block size (block must be 32)";
    case MX_ERR_DEVICE: return "HIP kernel launch failed";
    case MX_ERR_VALUE: return "a scalar argument is outside its range (attention scale: "
                              "positive, scale * log2(e) finite)";
    default: return "unknown status";
  }
}

mx_status mx_buffer_sizes(mx_format fmt, int block, int64_t rows, int64_t cols,
                          size_t* code_bytes, size_t* scale_bytes, size_t* aux_bytes) {
  bool nothing = false;
  mx_status st = check_common(fmt, block, rows, cols, &nothing);
  if (st != MX_OK) return st;
  const int64_t nb = nothing ? 0 : rows * (cols / MX_BLOCK);
  if (code_bytes) *code_bytes = (size_t)nb * (size_t)bytes_per_block(fmt);
  if (scale_bytes) *scale_bytes = (size_t)nb;
  if (aux_bytes) *aux_bytes = (fmt == MX_AXS6) ? (size_t)((nb + 3) / 4) : 0u;
  return MX_OK;
}

namespace {

// The argument checks of one quantize call; *nothing = true for an empty
// tensor (a no-op).
mx_status quantize_args(int fmt, int block, int in_dtype, const void* x, int64_t rows,
                        int64_t cols, const void* codes, const uint8_t* scales,
                        const uint8_t* aux, bool* nothing) {
  mx_status st = check_common(fmt, block, rows, cols, nothing);
  if (st != MX_OK) return st;
  if (!dtype_ok(in_dtype)) return MX_ERR_UNSUPPORTED;
  if (*nothing) return MX_OK;
  if (!x || !codes || !scales || (fmt == MX_AXS6 && !aux)) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes)) return MX_ERR_ALIGN;
  return MX_OK;
}

// One checked, non-empty tensor.
hipError_t quantize_one(int fmt, int in_dtype, const void* x, int64_t rows, int64_t cols,
                        void* codes, uint8_t* scales, uint8_t* aux, hipStream_t st) {
  const int64_t nb = rows * (cols / MX_BLOCK);
  if (is_exmy(fmt))
    return mxk::launch_exmy(0, exmy_width(fmt), exmy_params(fmt), in_dtype, x,
                            nullptr, nb, codes, scales, st);
  return mxk::launch_quantize(fmt, in_dtype, x, nb, codes, scales, aux, st);
}

}  // namespace

mx_status mx_quantize(mx_format fmt, int block, mx_dtype in_dtype, const void* x, int64_t rows,
                      int64_t cols, void* codes, uint8_t* scales, uint8_t* aux, void* stream) {
  bool nothing = false;
  const mx_status st = quantize_args(fmt, block, in_dtype, x, rows, cols, codes, scales, aux,
                                     &nothing);
  if (st != MX_OK || nothing) return st;
  if (forced_launch_failure()) return MX_ERR_DEVICE;
  return from_hip(quantize_one(fmt, in_dtype, x, rows, cols, codes, scales, aux,
                               static_cast<hipStream_t>(stream)));
}

mx_status mx_quantize_batch(mx_format fmt, int block, mx_dtype in_dtype,
                            const mx_tensor_desc* tensors, int count, void* stream) {
  if (count < 0) return MX_ERR_SHAPE;
  if (count > 0 && !tensors) return MX_ERR_NULL;
  // every tensor is checked before anything is enqueued
  int nonempty = 0;
  for (int i = 0; i < count; ++i) {
    const mx_tensor_desc& t = tensors[i];
    bool nothing = false;
    const mx_status st = quantize_args(fmt, block, in_dtype, t.x, t.rows, t.cols, t.codes,
                                       t.scales, t.aux, &nothing);
    if (st != MX_OK) return st;
    nonempty += nothing ? 0 : 1;
  }
  if (nonempty == 0) return MX_OK;
  if (forced_launch_failure()) return MX_ERR_DEVICE;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool grouped = fmt >= MX_FP6_E2M3 && fmt <= MX_FP8_E4M3;
  // MX hardware formats: up to kBatchMax tensors per launch, each tensor's
  // blocks in whole workgroups of 256; a launch stays under 2^31
  // workgroups, and a tensor too large for that goes alone
  constexpr int64_t kMaxWgs = 0x7FFFFFFF;
  mxk::QuantBatch a{};
  a.n = 0;
  a.wg_start[0] = 0;
  auto flush = [&]() -> hipError_t {
    if (a.n == 0) return hipSuccess;
    const hipError_t e = mxk::launch_quantize_batch(fmt, in_dtype, a, hs);
    a.n = 0;
    a.wg_start[0] = 0;
    return e;
  };
  for (int i = 0; i < count; ++i) {
    const mx_tensor_desc& t = tensors[i];
    if (t.rows == 0 || t.cols == 0) continue;
    const int64_t nb = t.rows * (t.cols / MX_BLOCK);
    const int64_t wgs = (nb + 255) / 256;
    if (!grouped || wgs > kMaxWgs / 2) {
      hipError_t e = flush();
      if (e == hipSuccess)
        e = quantize_one(fmt, in_dtype, t.x, t.rows, t.cols, t.codes, t.scales, t.aux, hs);
      if (e != hipSuccess) return MX_ERR_DEVICE;
      continue;
    }
    if (a.n == mxk::kBatchMax || (int64_t)a.wg_start[a.n] + wgs > kMaxWgs) {
      if (flush() != hipSuccess) return MX_ERR_DEVICE;
    }
    a.x[a.n] = t.x;
    a.codes[a.n] = t.codes;
    a.scales[a.n] = t.scales;
    a.nb[a.n] = nb;
    a.wg_start[a.n + 1] = (uint32_t)(a.wg_start[a.n] + wgs);
    ++a.n;
  }
  return from_hip(flush());
}

mx_status mx_dequantize(mx_format fmt, int block, const void* codes, const uint8_t* scales,
                        const uint8_t* aux, int64_t rows, int64_t cols, mx_dtype out_dtype,
                        void* y, void* stream) {
  bool nothing = false;
  mx_status st = check_common(fmt, block, rows, cols, &nothing);
  if (st != MX_OK) return st;
  if (!dtype_ok(out_dtype)) return MX_ERR_UNSUPPORTED;
  if (nothing) return MX_OK;
  if (!codes || !scales || !y || (fmt == MX_AXS6 && !aux)) return MX_ERR_NULL;
  if (!aligned16(codes) || !aligned16(y)) return MX_ERR_ALIGN;
  if (forced_launch_failure()) return MX_ERR_DEVICE;
  const int64_t nb = rows * (cols / MX_BLOCK);
  if (is_exmy(fmt))
    return from_hip(mxk::launch_exmy(1, exmy_width(fmt), exmy_params(fmt), out_dtype,
                                     codes, scales, nb, y, nullptr, static_cast<hipStream_t>(stream)));
  return from_hip(mxk::launch_dequantize(fmt, out_dtype, codes, scales, aux, nb, y,
                                         static_cast<hipStream_t>(stream)));
}

mx_status mx_fake_quantize(mx_format fmt, int block, mx_dtype dtype, const void* x, void* y,
                           int64_t rows, int64_t cols, void* stream) {
  bool nothing = false;
  mx_status st = check_common(fmt, block, rows, cols, &nothing);
  if (st != MX_OK) return st;
  if (!dtype_ok(dtype)) return MX_ERR_UNSUPPORTED;
  if (nothing) return MX_OK;
  if (!x || !y) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return MX_ERR_ALIGN;
  if (forced_launch_failure()) return MX_ERR_DEVICE;
  const int64_t nb = rows * (cols / MX_BLOCK);
  if (is_exmy(fmt))
    return from_hip(mxk::launch_exmy(2, exmy_width(fmt), exmy_params(fmt), dtype, x,
                                     nullptr, nb, y, nullptr, static_cast<hipStream_t>(stream)));
  return from_hip(mxk::launch_fake_quantize(fmt, dtype, x, nb, y,
                                            static_cast<hipStream_t>(stream)));
}

mx_status mx_softmax_quantize(mx_format fmt, int block, const float* s, int64_t rows,
                              int64_t cols, void* codes, uint8_t* scales, void* stream) {
  bool nothing = false;
  mx_status st = check_common(fmt, block, rows, cols, &nothing);
  if (st != MX_OK) return st;
  if (fmt == MX_AXS6 || is_exmy(fmt)) return MX_ERR_UNSUPPORTED;
  if (nothing) return MX_OK;
  if (!s || !codes || !scales) return MX_ERR_NULL;
  if (!aligned16(s) || !aligned16(codes)) return MX_ERR_ALIGN;
  if (forced_launch_failure()) return MX_ERR_DEVICE;
  return from_hip(mxk::launch_softmax_quantize(fmt, s, rows, cols, codes, scales,
                                               static_cast<hipStream_t>(stream)));
}

namespace {

mx_status attention(bool efq, mx_format v_fmt, int block, const void* q, const void* k,
                    const void* v_codes, const uint8_t* v_scales, int64_t heads, int64_t lq,
                    int64_t lk, int64_t d, float scale, mx_dtype out_dtype, void* o,
                    float* row_max, float* row_sum, void* p_codes, uint8_t* p_scales,
                    void* stream) {
  if (!(v_fmt == MX_FP8_E4M3 || v_fmt == MX_FP6_E2M3 || v_fmt == MX_FP6_E3M2 ||
        v_fmt == MX_FP4_E2M1))
    return MX_ERR_UNSUPPORTED;
  if (block != MX_BLOCK || d != 128 || (out_dtype != MX_BF16 && out_dtype != MX_FP32))
    return MX_ERR_UNSUPPORTED;
  if (heads < 0 || lq < 0 || lk <= 0 || lk % MX_BLOCK != 0) return MX_ERR_SHAPE;
  // int32 indices inside the kernel: every per-head and grid count must fit
  if (heads > INT32_MAX || lq > INT32_MAX - 128 || lk > (1 << 24)) return MX_ERR_SHAPE;
  if (heads * ((lq + 127) / 128) > INT32_MAX) return MX_ERR_SHAPE;
  if (heads > 0 && lq > 0 && (heads * lq > INT64_MAX / (2 * 128 * 16) ||
                              heads * lk > INT64_MAX / (2 * 128 * 16)))
    return MX_ERR_SHAPE;
  // the kernel takes the running maximum on the raw scores and scales it
  // by c = scale * log2(e), which orders the same only for c > 0
  const float c = scale * 0x1.715476p+0f;
  if (!(scale > 0.0f) || !(c < INFINITY)) return MX_ERR_VALUE;
  if ((p_codes == nullptr) != (p_scales == nullptr)) return MX_ERR_NULL;
  if (heads == 0 || lq == 0) return MX_OK;
  if (!q || !k || !v_codes || !v_scales || !o) return MX_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v_codes) || !aligned16(o) ||
      (p_codes && !aligned16(p_codes)))
    return MX_ERR_ALIGN;
  if (forced_launch_failure()) return MX_ERR_DEVICE;
  return from_hip(mxk::launch_attention(v_fmt, efq, out_dtype == MX_BF16, q, k, v_codes,
                                        v_scales, (int)heads, (int)lq, (int)lk, scale, o, row_max,
                                        row_sum, p_codes, p_scales,
                                        static_cast<hipStream_t>(stream)));
}

}  // namespace

mx_status mx_attention_fwd(mx_format v_fmt, int block, const void* q, const void* k,
                           const void* v_codes, const uint8_t* v_scales, int64_t heads,
                           int64_t lq, int64_t lk, int64_t d, float scale, mx_dtype out_dtype,
                           void* o, float* row_max, float* row_sum, void* p_codes,
                           uint8_t* p_scales, void* stream) {
  return attention(false, v_fmt, block, q, k, v_codes, v_scales, heads, lq, lk, d, scale,
                   out_dtype, o, row_max, row_sum, p_codes, p_scales, stream);
}

mx_status mx_attention_fwd_efq(mx_format v_fmt, int block, const void* q, const void* k,
                               const void* v_codes, const uint8_t* v_scales, int64_t heads,
                               int64_t lq, int64_t lk, int64_t d, float scale,
                               mx_dtype out_dtype, void* o, float* row_max, float* row_sum,
                               void* p_codes, uint8_t* p_scales, void* stream) {
  return attention(true, v_fmt, block, q, k, v_codes, v_scales, heads, lq, lk, d, scale,
                   out_dtype, o, row_max, row_sum, p_codes, p_scales, stream);
}

}  // extern "C"
