/*
 * mxref.h -- plain CPU oracle for block-shared-exponent (MX / AXS-6 /
 * eXmY) quantization, exp-then-quantize probabilities and the attention
 * forward with E2M1 probabilities.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the HIP library.
 *
 * Every function works on host memory, one block of 32 values at a time,
 * with exact double-precision arithmetic (a bf16/fp32 value divided by a
 * power of two is exact in double).  The rules it implements are stated in
 * mxref.c next to the code, each with the page passage it follows.
 *
 * Layouts (all row-major, contiguous):
 *   x        [rows, cols]          bf16 bit patterns (uint16) or fp32
 *   codes    [rows, cols/32, bpb]  packed element codes, bpb bytes/block
 *                                  (24 for FP6 and AXS-6, 16 for FP4,
 *                                  32 for FP8, 4w for eXmY of width w)
 *   scales   [rows, cols/32]       one E8M0 byte per block (AXS-6: the
 *                                  8-bit shared exponent, same encoding)
 *   aux      [ceil(nblocks/4)]     AXS-6 only: 2-bit config per block,
 *                                  block b at bits 2*(b%4).. of byte b/4
 */
#ifndef MXREF_H
#define MXREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MXREF_FP6_E2M3 = 0, MXREF_FP6_E3M2 = 1, MXREF_FP4_E2M1 = 2,
       MXREF_FP8_E4M3 = 3, MXREF_AXS6 = 4 };
enum { MXREF_BF16 = 0, MXREF_FP32 = 1, MXREF_F16 = 2 };
/* return codes: 0 ok, -1 bad argument */

int    mxref_bytes_per_block(int fmt);
/* value of one element code (sign included), before the block scale;
 * NaN for the E4M3 NaN codes */
double mxref_decode(int fmt, int code);
/* Q1+Q2: E8M0 byte of one block of n values (doubles) */
int    mxref_scale_byte(int fmt, const double *v, int n);
/* Q3: element code of v in a block whose scale byte is `byte` (!= 0xFF) */
int    mxref_encode(int fmt, double v, int byte);

int mxref_quantize(int fmt, int block, int in_dtype, const void *x,
                   int64_t rows, int64_t cols,
                   uint8_t *codes, uint8_t *scales, uint8_t *aux);
int mxref_dequantize(int fmt, int block, const uint8_t *codes,
                     const uint8_t *scales, const uint8_t *aux,
                     int64_t rows, int64_t cols, int out_dtype, void *y);
int mxref_fake_quantize(int fmt, int block, int dtype, const void *x, void *y,
                        int64_t rows, int64_t cols);

/* exp-then-quantize attention probabilities */
float mxref_exp(float d);
float mxref_exp2(float u);
int   mxref_exp2_n(const float *u, int64_t n, float *out);
int   mxref_softmax_probs(const float *s, int64_t rows, int64_t cols,
                          float *p);
int   mxref_softmax_quantize(int fmt, int block, const float *s,
                             int64_t rows, int64_t cols,
                             uint8_t *codes, uint8_t *scales);

/* attention forward: online softmax over kv_tile keys at a time, exp
 * (in base 2, mxref_exp2) then E2M1 quantization of the probabilities, V^T
 * block-quantized along the keys (layouts next to the definition in
 * mxref.c) */
int mxref_attention_fwd(int v_fmt, int block, const uint16_t *q,
                        const uint16_t *k, const uint8_t *v_codes,
                        const uint8_t *v_scales, int64_t heads, int64_t lq,
                        int64_t lk, int64_t d, float scale, int kv_tile,
                        int out_dtype, void *o, float *row_max,
                        float *row_sum, uint8_t *p_codes, uint8_t *p_scales);

/* EFQ's exp-free probabilities (a reading; parity unpinned by the pages):
 * the E2M1 codes of one block of 32 shifted scores, and the scale byte */
int mxref_efq_block(const float *dv, int *codes);
int mxref_efq_quantize_block(const float *dv, uint8_t *packed);
/* the same on shifted scores already in powers of two (u = d log2 e) */
int mxref_efq_block_log2(const float *u, int *codes);
/* the attention forward's form: raw scores s, c = fp32(scale log2 e), the
 * running maximum m of fp32(s c); the affine map as one fused multiply-add */
int mxref_efq_attention_block(const float *s, float c, float m, int *codes);
int mxref_efq_quantize_block_log2(const float *u, uint8_t *packed);
int mxref_attention_fwd_efq(int v_fmt, int block, const uint16_t *q,
                            const uint16_t *k, const uint8_t *v_codes,
                            const uint8_t *v_scales, int64_t heads,
                            int64_t lq, int64_t lk, int64_t d, float scale,
                            int kv_tile, int out_dtype, void *o,
                            float *row_max, float *row_sum, uint8_t *p_codes,
                            uint8_t *p_scales);

#ifdef __cplusplus
}
#endif
#endif
