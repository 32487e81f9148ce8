/*
 * mxref.c -- plain, slow, obviously-correct CPU oracle for block-shared-
 * exponent quantization (MXFP6 E2M3/E3M2, MXFP4 E2M1, MXFP8 E4M3, AXS-6 and
 * the generic eXmY formats), the exp-then-quantize probabilities, and the
 * attention forward whose probabilities are E2M1 blocks (exp-then-quantize,
 * or EFQ's exp-free rule).
 *
 * TEST INFRASTRUCTURE ONLY (see mxref.h).  Built with gcc -O2
 * -ffp-contract=off, no fast-math.  Every rule below cites the page it
 * follows; where the pages leave a step open the reading taken is named.
 *
 * Sources (titles of the pages):
 *   [AXS6]  "AXS-6: Adaptive eXponent Sharing" (pitchhut project page)
 *   [EXMY]  "eXmY: A Data Type and Technique for Arbitrary Bit Precision
 *            Quantization" (abstract)
 *   [EFQ]   "EFQ-Softmax: exp-free E2M1 probabilities" (explainer)
 *   [MXFP6] "Online MXFP6" (Sonar feature page)
 *
 * Parity pins: format tables, scale rule, RNE/saturation, packing and
 * dequantization are pinned by the CPU tests (library dtypes, brute-force
 * nearest-code search, closed-form invariants); the eXmY grids by field
 * enumeration, library dtypes and closed forms; the fixed exp and exp2 by
 * reference exponentials within their error bounds (and exp2's
 * coefficients by their definition); the attention forward by
 * closed forms (equal scores, a dominant key), brute-force probability
 * blocks and an error bound against exact attention.  The NaN/inf block
 * rule, the bit order inside a packed block and the AXS-6 element/config
 * semantics are readings of silent passages, and EFQ's affine rule is a
 * reading with no constants on the pages: parity unpinned by the pages,
 * pinned only by the written rules here and their unit tests.
 */
#include "mxref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element formats.                                                    */
/* [MXFP6] "Start a model" / "Select the FP6 encoding": OCP MXFP6 with  */
/* E2M3 (more mantissa) or E3M2 (more range), an E8M0 scale per 32.     */
/* [EFQ] "Jargon": E2M1 = 1 sign, 2 exponent, 1 mantissa bit.           */
/* [AXS6] "Overview": FP8 E4M3 has 1 sign, 4 exponent, 3 mantissa bits. */
/* Biases and ranges follow the OCP MX definitions the [MXFP6] page     */
/* invokes by name (a reading: the pages print no bias).                */
/* [AXS6] "Overview": a sign bit and 5 mantissa bits per value; read as  */
/* a uniform sign-magnitude grid m/16, m = 0..31, under the shared     */
/* exponent.                                                            */
/* ------------------------------------------------------------------ */
typedef struct {
  int bits;          /* code width including the sign bit */
  int ebits, mbits;  /* exponent and mantissa field widths */
  int bias;
  int emin;          /* unbiased exponent of the smallest normal */
  int emax;          /* floor(log2(largest finite value)) */
  double maxnorm;    /* largest finite magnitude */
  int nan_mag;       /* magnitude code meaning NaN, -1 if none */
  int fixed_point;   /* 1: magnitude m means m/16 (AXS-6) */
  int bpb;           /* packed bytes per 32-value block */
} fmt_t;

static const fmt_t FORMATS[5] = {
    /* E2M3 */ {6, 2, 3, 1, 0, 2, 7.5, -1, 0, 24},
    /* E3M2 */ {6, 3, 2, 3, -2, 4, 28.0, -1, 0, 24},
    /* E2M1 */ {4, 2, 1, 1, 0, 2, 6.0, -1, 0, 16},
    /* E4M3 */ {8, 4, 3, 7, -6, 8, 448.0, 0x7F, 0, 32},
    /* AXS6 */ {6, 0, 5, 0, 0, 0, 31.0 / 16.0, -1, 1, 24},
};

#define BLOCK 32

/* ------------------------------------------------------------------ */
/* Generic eXmY formats ([EXMY] abstract: every split of a bit width   */
/* into exponent and mantissa bits, e.g. e0m6 .. e6m0 for 7 bits).      */
/* Identifier 0x100 | e << 4 | m; width w = 1 + e + m, 3 <= w <= 9,     */
/* so e <= 8 (e8m0: zero and 2^-126 .. 2^128, whose largest magnitudes */
/* and scaled values lie beyond fp32; this code works in doubles).      */
/* Reading: sign-magnitude, IEEE-style fields with bias                 */
/* 2^(e-1) - 1 and subnormals, every code finite (no inf/NaN codes, as  */
/* in the OCP FP6/FP4 formats); e = 0 is a plain integer magnitude m.   */
/* ------------------------------------------------------------------ */
static int make_exmy(int e, int m, fmt_t *f) {
  int w = 1 + e + m;
  if (e < 0 || m < 0 || e > 8 || w < 3 || w > 9) return 0;
  f->bits = w;
  f->ebits = e;
  f->mbits = m;
  f->nan_mag = -1;
  f->fixed_point = 0;
  f->bpb = 4 * w;
  if (e >= 1) {
    f->bias = (1 << (e - 1)) - 1;
    f->emin = 1 - f->bias;
    f->emax = ((1 << e) - 1) - f->bias;                 /* top field is finite */
    f->maxnorm = ldexp(2.0 - ldexp(1.0, -m), f->emax);
  } else {
    f->bias = 0;
    f->emin = m;                  /* every magnitude is "subnormal": step 1 */
    f->emax = m - 1;
    f->maxnorm = ldexp(1.0, m) - 1.0;
  }
  return 1;
}

/* Fills *f for a format identifier; 0 if the identifier is unsupported. */
static int get_fmt(int fmt, fmt_t *f) {
  if (fmt >= 0 && fmt <= 4) {
    *f = FORMATS[fmt];
    return 1;
  }
  if ((fmt & ~0xFF) == 0x100) return make_exmy((fmt >> 4) & 0xF, fmt & 0xF, f);
  return 0;
}

int mxref_bytes_per_block(int fmt) {
  fmt_t f;
  return get_fmt(fmt, &f) ? f.bpb : -1;
}

/* floor(log2(a)) for a finite a > 0, exactly */
static int ilog2(double a) {
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  return e - 1;
}

/* ------------------------------------------------------------------ */
/* Decoding one code (sign included) to its unscaled value.            */
/* ------------------------------------------------------------------ */
double mxref_decode(int fmt, int code) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  int sign = (code >> (f->bits - 1)) & 1;
  int mag = code & ((1 << (f->bits - 1)) - 1);
  double v;
  if (f->nan_mag >= 0 && mag == f->nan_mag) return NAN;
  if (f->fixed_point) {
    v = mag / 16.0;
  } else {
    int e = mag >> f->mbits;
    int m = mag & ((1 << f->mbits) - 1);
    if (e == 0) /* subnormal: m * 2^(emin - mbits) */
      v = ldexp((double)m, f->emin - f->mbits);
    else        /* normal: (1 + m/2^mbits) * 2^(e - bias) */
      v = ldexp(1.0 + ldexp((double)m, -f->mbits), e - f->bias);
  }
  return sign ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Q1 + Q2: the shared scale of one block.                             */
/* [EFQ] article: the block scale is exponent-only and is chosen from  */
/* the largest magnitude inside the block; [EFQ] "Jargon": no other    */
/* block influences it.                                                 */
/* [MXFP6] "Start a model": an E8M0 scale per block of 32 values.      */
/* Reading (OCP conversion rule): byte = floor(log2 amax) - emax + 127,*/
/* clamped to 0..254; amax == 0 gives byte 0; any NaN or inf in the    */
/* block gives 0xFF, E8M0's NaN (the element formats hold neither).    */
/* AXS-6 uses the same rule with emax = 0 ([AXS6] "Overview": one      */
/* 8-bit shared exponent per 32 values).                                */
/* ------------------------------------------------------------------ */
int mxref_scale_byte(int fmt, const double *v, int n) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  double amax = 0.0;
  int i, b;
  for (i = 0; i < n; i++) /* Q1: classify */
    if (isnan(v[i]) || isinf(v[i])) return 0xFF;
  for (i = 0; i < n; i++) /* Q2: absolute maximum */
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  if (amax == 0.0) return 0;
  b = ilog2(amax) - f->emax + 127;
  if (b < 0) b = 0;
  if (b > 254) b = 254;
  return b;
}

/* ------------------------------------------------------------------ */
/* Q3: one element.                                                    */
/* a = |v| / 2^(byte-127) (exact); a is clamped to the largest finite  */
/* magnitude (saturation, never NaN from a finite input); the code is  */
/* the grid point nearest to a, and on an exact tie the code whose     */
/* last bit is 0 (round-to-nearest-even on the codes); the sign bit is */
/* copied, so -0 and negative values that round to zero keep it.       */
/* ------------------------------------------------------------------ */

/* magnitude code of a grid value r (r >= 0 on the grid of f) */
static int code_of_value(const fmt_t *f, double r) {
  if (r < ldexp(1.0, f->emin)) /* subnormal code (every code when e = 0) */
    return (int)(r / ldexp(1.0, f->emin - f->mbits));
  {
    int er = ilog2(r);
    int mant = (int)((r / ldexp(1.0, er) - 1.0) * (double)(1 << f->mbits));
    return ((er + f->bias) << f->mbits) | mant;
  }
}

int mxref_encode(int fmt, double v, int byte) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  double X = ldexp(1.0, byte - 127);
  double a = fabs(v) / X;
  int sign = signbit(v) ? 1 : 0;
  int mag;
  if (a > f->maxnorm) a = f->maxnorm;
  if (f->fixed_point) {
    mag = (int)nearbyint(a * 16.0); /* step 1/16, RNE */
    if (mag > 31) mag = 31;
  } else if (a == 0.0) {
    mag = 0;
  } else {
    int ea = ilog2(a);
    int eu = ea > f->emin ? ea : f->emin;       /* binade of the step */
    double u = ldexp(1.0, eu - f->mbits);       /* grid step at a */
    double nlo = floor(a / u);                  /* a / u is exact */
    double rlo = nlo * u, rhi = (nlo + 1.0) * u; /* neighbouring grid values */
    int clo = code_of_value(f, rlo), chi = code_of_value(f, rhi);
    if (a - rlo < rhi - a) mag = clo;
    else if (a - rlo > rhi - a) mag = chi;
    else mag = (clo % 2 == 0) ? clo : chi;      /* tie: the even code */
  }
  return (sign << (f->bits - 1)) | mag;
}

/* ------------------------------------------------------------------ */
/* Q4: packing of one block's 32 codes.                                */
/* [EXMY] abstract: codes whose width is not a power of two are packed */
/* densely while staying byte addressable; [MXFP6] "Start a model":    */
/* six-bit codes, packed.  Reading: the codes form a little-endian bit */
/* stream, code k at stream bits [k*w, k*w + w), stream bit s in bit   */
/* s%8 of byte s/8.                                                    */
/* For 6-bit codes every 4 codes fill 3 bytes; 4-bit codes put the     */
/* even element in the low nibble; 8-bit codes are one per byte.       */
/* ------------------------------------------------------------------ */
static void pack_block(const fmt_t *f, const int *c, uint8_t *out) {
  int k, j;
  memset(out, 0, (size_t)f->bpb);
  for (k = 0; k < BLOCK; k++)
    for (j = 0; j < f->bits; j++) {
      int s = k * f->bits + j;
      if ((c[k] >> j) & 1) out[s / 8] |= (uint8_t)(1u << (s % 8));
    }
}

static void unpack_block(const fmt_t *f, const uint8_t *in, int *c) {
  int k, j;
  for (k = 0; k < BLOCK; k++) {
    c[k] = 0;
    for (j = 0; j < f->bits; j++) {
      int s = k * f->bits + j;
      c[k] |= ((in[s / 8] >> (s % 8)) & 1) << j;
    }
  }
}

/* ------------------------------------------------------------------ */
/* Host number formats: bf16 = top half of an fp32 bit pattern; fp16 =  */
/* IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10 mantissa     */
/* bits, subnormals), the other source type the [MXFP6] page names      */
/* ("Start a model": BF16 or FP16 weights).                             */
/* ------------------------------------------------------------------ */
static double half_to_double(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -24);          /* m * 2^-24 */
  else
    v = ldexp(1024.0 + m, e - 25);      /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static double load_value(int dtype, const void *x, int64_t i) {
  uint32_t u;
  float fv;
  if (dtype == MXREF_F16) return half_to_double(((const uint16_t *)x)[i]);
  if (dtype == MXREF_BF16)
    u = (uint32_t)((const uint16_t *)x)[i] << 16;
  else
    memcpy(&u, (const float *)x + i, 4);
  memcpy(&fv, &u, 4);
  return (double)fv;
}

/* Round a double to a binary format with p significand bits (hidden bit
 * included) and normal exponents emin..emax, round-to-nearest-even,
 * gradual underflow, overflow to infinity; return the IEEE bit pattern of
 * the fp32 container (bf16 = top 16 bits).  NaN -> canonical quiet NaN. */
static uint32_t round_to_bits(double y, int p) {
  const int emin = -126, emax = 127;
  uint32_t sign = signbit(y) ? 0x80000000u : 0u;
  double ay = fabs(y), n, r;
  int e, q;
  uint32_t field, mant;
  if (isnan(y)) return 0x7FC00000u;
  if (ay == 0.0) return sign;
  if (isinf(y)) return sign | 0x7F800000u;
  e = ilog2(ay);
  q = (e > emin ? e : emin) - (p - 1); /* exponent of one ulp */
  n = nearbyint(ay / ldexp(1.0, q));
  r = n * ldexp(1.0, q);
  if (r >= ldexp(1.0, emax + 1)) return sign | 0x7F800000u;
  if (r < ldexp(1.0, emin)) {
    field = 0;
    mant = (uint32_t)(r / ldexp(1.0, emin - (p - 1)));
  } else {
    int er = ilog2(r);
    field = (uint32_t)(er + 127);
    mant = (uint32_t)((r / ldexp(1.0, er) - 1.0) * ldexp(1.0, p - 1));
  }
  return sign | (field << 23) | (mant << (24 - p));
}

/* Round a double to binary16 (11 significand bits, normal exponents
 * -14..15), round-to-nearest-even, gradual underflow down to 2^-24,
 * overflow to infinity; NaN -> the canonical quiet NaN 0x7E00. */
static uint16_t round_to_half(double y) {
  const uint16_t sign = signbit(y) ? 0x8000u : 0u;
  double ay = fabs(y), r;
  int e, q;
  if (isnan(y)) return 0x7E00u;
  if (ay == 0.0) return sign;
  if (isinf(y)) return (uint16_t)(sign | 0x7C00u);
  e = ilog2(ay);
  q = (e > -14 ? e : -14) - 10; /* exponent of one ulp */
  r = nearbyint(ay / ldexp(1.0, q)) * ldexp(1.0, q);
  if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u);
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  {
    int er = ilog2(r);
    uint16_t field = (uint16_t)(er + 15);
    uint16_t mant = (uint16_t)((r / ldexp(1.0, er) - 1.0) * 1024.0);
    return (uint16_t)(sign | (field << 10) | mant);
  }
}

static void store_value(int dtype, void *y, int64_t i, double v) {
  if (dtype == MXREF_F16) {
    ((uint16_t *)y)[i] = round_to_half(v);
  } else if (dtype == MXREF_BF16) {
    uint32_t u = round_to_bits(v, 8);
    ((uint16_t *)y)[i] = (uint16_t)(u >> 16);
  } else {
    uint32_t u = round_to_bits(v, 24);
    memcpy((float *)y + i, &u, 4);
  }
}

static int check_args(int fmt, int block, int64_t rows, int64_t cols) {
  fmt_t f;
  if (!get_fmt(fmt, &f) || block != BLOCK) return -1;
  if (rows < 0 || cols < 0 || cols % BLOCK) return -1;
  return 0;
}

/* one block: Q1-Q3 on 32 doubles, codes into c[] */
static int quantize_values(const fmt_t *f, int fmt, const double *v, int *c) {
  int k, byte = mxref_scale_byte(fmt, v, BLOCK);
  for (k = 0; k < BLOCK; k++)
    c[k] = (byte == 0xFF) ? 0 : mxref_encode(fmt, v[k], byte);
  (void)f;
  return byte;
}

static int dtype_ok(int d) { return d == MXREF_BF16 || d == MXREF_FP32 || d == MXREF_F16; }

int mxref_quantize(int fmt, int block, int in_dtype, const void *x,
                   int64_t rows, int64_t cols, uint8_t *codes,
                   uint8_t *scales, uint8_t *aux) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  int64_t nb, b;
  double v[BLOCK];
  int c[BLOCK], k;
  if (check_args(fmt, block, rows, cols) || !dtype_ok(in_dtype)) return -1;
  nb = rows * (cols / BLOCK);
  for (b = 0; b < nb; b++) {
    for (k = 0; k < BLOCK; k++) v[k] = load_value(in_dtype, x, b * BLOCK + k);
    scales[b] = (uint8_t)quantize_values(f, fmt, v, c);
    pack_block(f, c, codes + b * f->bpb);
  }
  /* [AXS6] "Overview": a 2-bit config field once per block.  Reading: the
   * only configuration defined here is 0 (the uniform grid above). */
  if (fmt == MXREF_AXS6)
    for (b = 0; b < (nb + 3) / 4; b++) aux[b] = 0;
  return 0;
}

/* ------------------------------------------------------------------ */
/* D: dequantize.  y = sign * decode(mag) * 2^(byte-127), exact, then  */
/* rounded to the output type (RNE).  Byte 0xFF, an E4M3 NaN code, or  */
/* an AXS-6 block whose config is not 0 decodes to canonical NaN.       */
/* ------------------------------------------------------------------ */
int mxref_dequantize(int fmt, int block, const uint8_t *codes,
                     const uint8_t *scales, const uint8_t *aux, int64_t rows,
                     int64_t cols, int out_dtype, void *y) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  int64_t nb, b;
  int c[BLOCK], k;
  if (check_args(fmt, block, rows, cols) || !dtype_ok(out_dtype)) return -1;
  nb = rows * (cols / BLOCK);
  for (b = 0; b < nb; b++) {
    int byte = scales[b];
    int poisoned = (byte == 0xFF);
    if (fmt == MXREF_AXS6 && ((aux[b / 4] >> (2 * (b % 4))) & 3) != 0)
      poisoned = 1;
    unpack_block(f, codes + b * f->bpb, c);
    for (k = 0; k < BLOCK; k++) {
      double val = poisoned ? NAN : mxref_decode(fmt, c[k]) * ldexp(1.0, byte - 127);
      store_value(out_dtype, y, b * BLOCK + k, val);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* F: fake-quantize = dequantize(quantize(x)) in the input type, one   */
/* block at a time with no packed intermediate ([AXS6] "Quick Start":  */
/* a fused fake-quantize call over 32-value blocks that allocates no   */
/* intermediate buffer).                                                */
/* ------------------------------------------------------------------ */
int mxref_fake_quantize(int fmt, int block, int dtype, const void *x, void *y,
                        int64_t rows, int64_t cols) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  int64_t nb, b;
  double v[BLOCK];
  int c[BLOCK], k, byte;
  if (check_args(fmt, block, rows, cols) || !dtype_ok(dtype)) return -1;
  nb = rows * (cols / BLOCK);
  for (b = 0; b < nb; b++) {
    for (k = 0; k < BLOCK; k++) v[k] = load_value(dtype, x, b * BLOCK + k);
    byte = quantize_values(f, fmt, v, c);
    for (k = 0; k < BLOCK; k++) {
      double val = (byte == 0xFF) ? NAN : mxref_decode(fmt, c[k]) * ldexp(1.0, byte - 127);
      store_value(dtype, y, b * BLOCK + k, val);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* X: exp-then-quantize attention probabilities.                       */
/* [EFQ] "Jargon" (shifted scores, exp-then-quantize) and the article: */
/* subtract the row maximum, evaluate exp() in higher precision,       */
/* materialize the probability block, then quantize it to block-scaled */
/* E2M1.  Reading: "higher precision" is fp32 through the fixed op     */
/* sequence mxref_exp below, so that a quantized code never depends on */
/* which exp library ran.                                               */
/* ------------------------------------------------------------------ */

/* Cody-Waite range reduction (W. J. Cody and W. Waite, "Software Manual
 * for the Elementary Functions", 1980) with a degree-7 Taylor polynomial:
 *   n = rint(d * log2(e)),  r = d - n*ln2 (ln2 split in a 16-bit head and
 *   a tail, each step one fused multiply-add),  p = sum_{k<=7} r^k / k!
 *   by Horner's rule with fused multiply-adds,  exp(d) = p * 2^n.
 * Constants: log2(e), ln2 and 1/k! each rounded to fp32; the head of ln2
 * is ln2's fp32 significand cut to its top 16 bits, the tail is the fp32
 * rounding of the remainder.  2^n is applied by exact multiplications by
 * powers of two (two of them when 2^n alone is not a normal fp32), so the
 * only rounding of the scaling is that of the final product. */
float mxref_exp(float d) {
  const float LOG2E = 0x1.715476p+0f;
  const float LN2_HI = 0x1.62e400p-1f;
  const float LN2_LO = 0x1.7f7d1cp-20f;
  const float C2 = 0x1.000000p-1f, C3 = 0x1.555556p-3f, C4 = 0x1.555556p-5f,
              C5 = 0x1.111112p-7f, C6 = 0x1.6c16c2p-10f, C7 = 0x1.a01a02p-13f;
  float nf, r, p;
  int n;
  if (isnan(d)) return d;
  if (d > 88.75f) return INFINITY;
  if (d < -104.0f) return 0.0f;
  nf = rintf(d * LOG2E);
  r = fmaf(-nf, LN2_HI, d);
  r = fmaf(-nf, LN2_LO, r);
  p = C7;
  p = fmaf(p, r, C6);
  p = fmaf(p, r, C5);
  p = fmaf(p, r, C4);
  p = fmaf(p, r, C3);
  p = fmaf(p, r, C2);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  n = (int)nf;
  if (n < -100) { p = p * 0x1p-50f; n += 50; }
  if (n > 100) { p = p * 0x1p+50f; n -= 50; }
  return p * ldexpf(1.0f, n);
}

/* 2^u, for the attention forward's probabilities (attention_fwd below
 * evaluates exp(t - m) as 2^((t - m) log2 e) with log2 e joined to the
 * score scale):
 *   n = rint(u),  f = u - n (exact, |f| <= 1/2),
 *   p = 1 + c1 f + ... + c5 f^5 by Horner's rule with fused multiply-adds,
 *   2^u = p * 2^n with one rounding (exact multiplications by powers of two
 *   as in mxref_exp).
 * c1..c5 minimize the largest relative error of 1 + f (c1 + ... + c5 f^4)
 * against 2^f over [-1/2, 1/2] (a linear program on a dense grid; the
 * constant term is held at 1, so 2^u is exact for every integer u in
 * [-149, 0]), each then moved by a few fp32 ulps to the values whose fp32
 * evaluation errs least.  The result is within 2.1 ulp of 2^u. */
float mxref_exp2(float u) {
  const float C1 = 0x1.62e42ap-1f, C2 = 0x1.ebf994p-3f, C3 = 0x1.c6b5acp-5f,
              C4 = 0x1.3cf68ap-7f, C5 = 0x1.5c54b4p-10f;
  float nf, f, p;
  int n;
  if (isnan(u)) return u;
  if (u > 128.0f) return INFINITY;
  if (u < -151.0f) return 0.0f;
  nf = rintf(u);
  f = u - nf;
  p = C5;
  p = fmaf(p, f, C4);
  p = fmaf(p, f, C3);
  p = fmaf(p, f, C2);
  p = fmaf(p, f, C1);
  p = fmaf(p, f, 1.0f);
  n = (int)nf;
  if (n < -100) { p = p * 0x1p-50f; n += 50; }
  if (n > 100) { p = p * 0x1p+50f; n -= 50; }
  return p * ldexpf(1.0f, n);
}

/* mxref_exp2 over an array (for the tests' dense sweeps) */
int mxref_exp2_n(const float *u, int64_t n, float *out) {
  int64_t i;
  if (n < 0) return -1;
  for (i = 0; i < n; i++) out[i] = mxref_exp2(u[i]);
  return 0;
}

/* P = exp(s - rowmax) per row.  The row maximum is exact; a NaN anywhere
 * in the row makes it NaN.  d = s - rowmax is one fp32 subtraction. */
int mxref_softmax_probs(const float *s, int64_t rows, int64_t cols, float *p) {
  int64_t r, i;
  if (rows < 0 || cols < 0) return -1;
  for (r = 0; r < rows; r++) {
    const float *row = s + r * cols;
    float m = -INFINITY;
    int has_nan = 0;
    for (i = 0; i < cols; i++) {
      if (isnan(row[i])) has_nan = 1;
      else if (row[i] > m) m = row[i];
    }
    if (has_nan) m = NAN;
    for (i = 0; i < cols; i++) {
      float d = row[i] - m;
      p[r * cols + i] = mxref_exp(d);
    }
  }
  return 0;
}

int mxref_softmax_quantize(int fmt, int block, const float *s, int64_t rows,
                           int64_t cols, uint8_t *codes, uint8_t *scales) {
  fmt_t fs;
  const fmt_t *f = get_fmt(fmt, &fs) ? &fs : 0;
  int64_t r, j, nbr;
  double v[BLOCK];
  int c[BLOCK], k;
  float prow[BLOCK];
  if (check_args(fmt, block, rows, cols) || fmt == MXREF_AXS6) return -1;
  nbr = cols / BLOCK;
  for (r = 0; r < rows; r++) {
    const float *row = s + r * cols;
    float m = -INFINITY;
    int has_nan = 0;
    int64_t i;
    for (i = 0; i < cols; i++) {
      if (isnan(row[i])) has_nan = 1;
      else if (row[i] > m) m = row[i];
    }
    if (has_nan) m = NAN;
    for (j = 0; j < nbr; j++) {
      int64_t b = r * nbr + j;
      for (k = 0; k < BLOCK; k++) {
        float d = row[j * BLOCK + k] - m;
        prow[k] = mxref_exp(d);
        v[k] = (double)prow[k];
      }
      scales[b] = (uint8_t)quantize_values(f, fmt, v, c);
      pack_block(f, c, codes + b * f->bpb);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Attention forward with exp-then-quantize probabilities.             */
/* [EFQ] "Does it change FlashAttention?" and the stage table: the     */
/* online softmax keeps a running row maximum, rescales the earlier    */
/* partial sums when it grows, accumulates in high precision and       */
/* normalizes once at the end; the probabilities are produced by exp() */
/* of the shifted scores and quantized to block-scaled E2M1 (MXFP4)     */
/* before the PV product; [EFQ] stage table, "Denominator operand":    */
/* the E2M1 block also feeds the denominator (the conventional path    */
/* leaves this open; reading: the same operand, as in the EFQ path).   */
/* Readings where the pages are silent:                                */
/*  - scores s = q . k from bf16 q, k, summed in double and rounded     */
/*    once to fp32;                                                     */
/*  - exp is evaluated in base 2: c = fp32(scale * log2 e) and          */
/*    t = fp32(s * c), the scaled score in powers of two, so that       */
/*    exp(s scale - max) = 2^(t - max t) (rounding aside);              */
/*  - the running maximum of t is updated once per kv_tile keys (NaN   */
/*    scores are skipped by the maximum, as fmax does); alpha =        */
/*    mxref_exp2(m_old - m_new) rescales the sums only when m grows;   */
/*  - p = mxref_exp2(fp32(t - m_new)), quantized per 32 keys to E2M1   */
/*    by the MX rules above (a NaN p poisons its block, so the row's    */
/*    output is NaN);                                                   */
/*  - V arrives transposed and block-quantized along the keys (V^T as  */
/*    [d, lk] in any MX element format), and is decoded exactly;        */
/*  - l and the numerator are accumulated in double from the decoded   */
/*    E2M1 values; o = numerator / l, rounded once to the output type. */
/* Layouts: q [heads, lq, d], k [heads, lk, d] (bf16 bits); v_codes    */
/* [heads, d, lk/32, bpb], v_scales [heads, d, lk/32]; o [heads, lq,   */
/* d]; row_max, row_sum [heads, lq] (the row's largest fp32(s * scale) */
/* in natural units, NaN scores skipped, and fp32(l));                  */
/* p_codes [heads, lq, lk/32, 16], p_scales [heads, lq, lk/32]: the    */
/* E2M1 blocks as they entered the PV product.  The last four may be   */
/* NULL.                                                                */
/* ------------------------------------------------------------------ */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float fv;
  memcpy(&fv, &u, 4);
  return (double)fv;
}

/* ------------------------------------------------------------------ */
/* EFQ's exp-free probability block ([EFQ] article, the paragraph that  */
/* starts "Concretely", and the stage table): no exp(); an exponent-     */
/* only scale taken from the largest value in the block normalizes the */
/* shifted scores, and a single affine rule turns them into unsigned     */
/* codes.  The pages give no constants, so the rule below is a reading  */
/* (PARITY UNPINNED by the pages; only its stated properties are       */
/* tested):                                                             */
/*   u = fp32(d * log2 e)             shifted score in powers of two    */
/*                                    (the attention forward hands in   */
/*                                    its base-2 t - m directly)        */
/*   U = max u; byte = clamp(floor(U) - 2 + 127, 0, 254)                */
/*                                    (the MX rule applied to 2^U)      */
/*   w = u - (byte - 127)             exact in fp32                     */
/*   code = trunc(clamp(fp32(fma(w, 2, 2.5)), 0, 7.5))                  */
/* so w = 0, 1, 2 (values X, 2X, 4X) give the even codes 2, 4, 6 that   */
/* hold exactly those values, and the odd codes take the log-domain     */
/* midpoints.  A NaN shifted score poisons the block (0xFF, codes 0);   */
/* U = -inf gives byte 0 and codes 0.                                   */
/* ------------------------------------------------------------------ */
int mxref_efq_block_log2(const float *u, int *codes) {
  float U = -INFINITY;
  int k, byte, E;
  for (k = 0; k < BLOCK; k++)
    if (isnan(u[k])) {
      for (k = 0; k < BLOCK; k++) codes[k] = 0;
      return 0xFF;
    }
  for (k = 0; k < BLOCK; k++)
    if (u[k] > U) U = u[k];
  if (U == -INFINITY) {
    for (k = 0; k < BLOCK; k++) codes[k] = 0;
    return 0;
  }
  /* every U below -1000 gives byte 0 too (and keeps floor in int range) */
  E = (int)floorf(U < -1000.0f ? -1000.0f : U);
  byte = E - 2 + 127;
  if (byte < 0) byte = 0;
  if (byte > 254) byte = 254;
  for (k = 0; k < BLOCK; k++) {
    float w = u[k] - (float)(byte - 127);
    float x = fmaf(w, 2.0f, 2.5f);
    if (!(x > 0.0f)) x = 0.0f;
    if (x > 7.5f) x = 7.5f;
    codes[k] = (int)x;
  }
  return byte;
}

/* EFQ inside the attention forward: the scale byte as in
 * mxref_efq_block_log2 from u = fp32(fp32(s c) - m), and the affine map
 * 2 (u - (byte - 127)) + 2.5 evaluated from the raw fp32 score s in one
 * fused multiply-add, a = fma(s, 2c, fp32((2.5 - 2 (byte - 127)) - 2m))
 * (the same exact value before rounding, with fewer roundings);
 * code = trunc(clamp(a, 0, 7.5)). */
int mxref_efq_attention_block(const float *s, float c, float m, int *codes) {
  float u[BLOCK], U = -INFINITY, k2, a;
  int k, byte, E;
  for (k = 0; k < BLOCK; k++) {
    u[k] = s[k] * c - m;
    if (isnan(u[k])) {
      for (k = 0; k < BLOCK; k++) codes[k] = 0;
      return 0xFF;
    }
  }
  for (k = 0; k < BLOCK; k++)
    if (u[k] > U) U = u[k];
  if (U == -INFINITY) {
    for (k = 0; k < BLOCK; k++) codes[k] = 0;
    return 0;
  }
  E = (int)floorf(U < -1000.0f ? -1000.0f : U);
  byte = E - 2 + 127;
  if (byte < 0) byte = 0;
  if (byte > 254) byte = 254;
  k2 = (2.5f - 2.0f * (float)(byte - 127)) - 2.0f * m;
  for (k = 0; k < BLOCK; k++) {
    a = fmaf(s[k], 2.0f * c, k2);
    if (!(a > 0.0f)) a = 0.0f;
    if (a > 7.5f) a = 7.5f;
    codes[k] = (int)a;
  }
  return byte;
}

int mxref_efq_block(const float *dv, int *codes) {
  const float LOG2E = 0x1.715476p+0f;
  float u[BLOCK];
  int k;
  for (k = 0; k < BLOCK; k++) u[k] = dv[k] * LOG2E;
  return mxref_efq_block_log2(u, codes);
}

int mxref_efq_quantize_block_log2(const float *u, uint8_t *packed) {
  fmt_t fp;
  int codes[BLOCK], byte;
  get_fmt(MXREF_FP4_E2M1, &fp);
  byte = mxref_efq_block_log2(u, codes);
  pack_block(&fp, codes, packed);
  return byte;
}

int mxref_efq_quantize_block(const float *dv, uint8_t *packed) {
  const float LOG2E = 0x1.715476p+0f;
  float u[BLOCK];
  int k;
  for (k = 0; k < BLOCK; k++) u[k] = dv[k] * LOG2E;
  return mxref_efq_quantize_block_log2(u, packed);
}

static int attention_fwd(int rule, int v_fmt, int block, const uint16_t *q,
                         const uint16_t *k, const uint8_t *v_codes,
                         const uint8_t *v_scales, int64_t heads, int64_t lq,
                         int64_t lk, int64_t d, float scale, int kv_tile,
                         int out_dtype, void *o, float *row_max,
                         float *row_sum, uint8_t *p_codes, uint8_t *p_scales) {
  const float LOG2E = 0x1.715476p+0f;
  fmt_t fv, fp;
  int64_t h, i, j, c, kk, nbk;
  float c2;
  double *vhat = 0, *acc = 0;
  float *t = 0, *sr = 0;
  if (!get_fmt(v_fmt, &fv) || v_fmt == MXREF_AXS6 || (v_fmt & ~0xFF)) return -1;
  get_fmt(MXREF_FP4_E2M1, &fp);
  if (block != BLOCK || heads < 0 || lq < 0 || d <= 0 || lk <= 0 ||
      lk % BLOCK || kv_tile <= 0 || kv_tile % BLOCK)
    return -1;
  /* the scale must be positive with scale * log2 e finite */
  c2 = scale * LOG2E;
  if (!(scale > 0.0f) || !(c2 < INFINITY)) return -1;
  nbk = lk / BLOCK;
  vhat = (double *)malloc(sizeof(double) * (size_t)(d * lk));
  acc = (double *)malloc(sizeof(double) * (size_t)d);
  t = (float *)malloc(sizeof(float) * (size_t)lk);
  sr = (float *)malloc(sizeof(float) * (size_t)lk);
  if (!vhat || !acc || !t || !sr) {
    free(vhat); free(acc); free(t); free(sr);
    return -1;
  }
  for (h = 0; h < heads; h++) {
    /* decode V^T of this head: vhat[c * lk + key] */
    for (c = 0; c < d; c++)
      for (j = 0; j < nbk; j++) {
        int64_t b = (h * d + c) * nbk + j;
        int codes[BLOCK], e;
        int byte = v_scales[b];
        unpack_block(&fv, v_codes + b * fv.bpb, codes);
        for (e = 0; e < BLOCK; e++)
          vhat[c * lk + j * BLOCK + e] =
              byte == 0xFF ? NAN
                           : mxref_decode(v_fmt, codes[e]) * ldexp(1.0, byte - 127);
      }
    for (i = 0; i < lq; i++) {
      const uint16_t *qi = q + (h * lq + i) * d;
      float m = -INFINITY, row_top = -INFINITY;
      double l = 0.0;
      int64_t row = h * lq + i;
      /* scores of the whole row in powers of two, t = fp32(fp32(q . k) * c2),
       * and the largest fp32(fp32(q . k) * scale) */
      for (kk = 0; kk < lk; kk++) {
        const uint16_t *kr = k + (h * lk + kk) * d;
        double s = 0.0;
        for (c = 0; c < d; c++) s += bf16_value(qi[c]) * bf16_value(kr[c]);
        sr[kk] = (float)s;
        t[kk] = sr[kk] * c2;
        if ((float)s * scale > row_top) row_top = (float)s * scale;
      }
      for (c = 0; c < d; c++) acc[c] = 0.0;
      for (j = 0; j < lk; j += kv_tile) {
        int64_t end = j + kv_tile < lk ? j + kv_tile : lk;
        float m_new = m;
        for (kk = j; kk < end; kk++)
          if (t[kk] > m_new) m_new = t[kk]; /* NaN never compares greater */
        if (m_new > m) {
          double alpha = (double)mxref_exp2(m - m_new);
          l *= alpha;
          for (c = 0; c < d; c++) acc[c] *= alpha;
          m = m_new;
        }
        for (kk = j; kk < end; kk += BLOCK) {
          double pv[BLOCK], phat[BLOCK];
          float dv[BLOCK];
          int codes[BLOCK], e, byte;
          for (e = 0; e < BLOCK; e++) dv[e] = t[kk + e] - m;
          if (rule == 0) {
            for (e = 0; e < BLOCK; e++) pv[e] = (double)mxref_exp2(dv[e]);
            byte = quantize_values(&fp, MXREF_FP4_E2M1, pv, codes);
          } else {
            byte = mxref_efq_attention_block(sr + kk, c2, m, codes);
          }
          for (e = 0; e < BLOCK; e++)
            phat[e] = byte == 0xFF ? NAN
                                   : mxref_decode(MXREF_FP4_E2M1, codes[e]) *
                                         ldexp(1.0, byte - 127);
          if (p_codes) pack_block(&fp, codes, p_codes + (row * nbk + kk / BLOCK) * fp.bpb);
          if (p_scales) p_scales[row * nbk + kk / BLOCK] = (uint8_t)byte;
          for (e = 0; e < BLOCK; e++) {
            l += phat[e];
            for (c = 0; c < d; c++) acc[c] += phat[e] * vhat[c * lk + kk + e];
          }
        }
      }
      for (c = 0; c < d; c++) store_value(out_dtype, o, row * d + c, acc[c] / l);
      if (row_max) row_max[row] = row_top;
      if (row_sum) row_sum[row] = (float)l;
    }
  }
  free(vhat);
  free(acc);
  free(t);
  free(sr);
  return 0;
}

int mxref_attention_fwd(int v_fmt, int block, const uint16_t *q,
                        const uint16_t *k, const uint8_t *v_codes,
                        const uint8_t *v_scales, int64_t heads, int64_t lq,
                        int64_t lk, int64_t d, float scale, int kv_tile,
                        int out_dtype, void *o, float *row_max,
                        float *row_sum, uint8_t *p_codes, uint8_t *p_scales) {
  return attention_fwd(0, v_fmt, block, q, k, v_codes, v_scales, heads, lq, lk,
                       d, scale, kv_tile, out_dtype, o, row_max, row_sum,
                       p_codes, p_scales);
}

/* the same forward with EFQ's exp-free probability blocks (a reading,
 * parity unpinned by the pages; see mxref_efq_block and, for the form used
 * here, mxref_efq_attention_block) */
int mxref_attention_fwd_efq(int v_fmt, int block, const uint16_t *q,
                            const uint16_t *k, const uint8_t *v_codes,
                            const uint8_t *v_scales, int64_t heads,
                            int64_t lq, int64_t lk, int64_t d, float scale,
                            int kv_tile, int out_dtype, void *o,
                            float *row_max, float *row_sum, uint8_t *p_codes,
                            uint8_t *p_scales) {
  return attention_fwd(1, v_fmt, block, q, k, v_codes, v_scales, heads, lq, lk,
                       d, scale, kv_tile, out_dtype, o, row_max, row_sum,
                       p_codes, p_scales);
}
