// mx_kernels.hip -- gfx950 kernels for block-shared-exponent quantization.
//
// Layout: one lane owns one 32-value block.  The lane reads its block (64 B
// of bf16 or fp16, 128 B of fp32) with 128-bit loads, reduces the largest
// magnitude in registers, derives the shared scale byte, converts the 32
// values with the scaled-convert instructions (FP6: one 32-wide instruction;
// FP4/FP8: one per pair) or, for AXS-6, with integer/fp32 arithmetic, and
// writes its packed codes (24/16/32 B) and its scale byte.  No arithmetic
// crosses lanes, so every output byte has exactly one writer.  Wide outputs,
// and the 16-bit inputs of the MX quantizers and of the MX and AXS-6
// fake-quantizers, pass through a per-wave LDS tile of 64 blocks for
// coalesced 1 KB accesses; a wave has read its whole tile before it writes
// any of it, so in-place fake-quantization is safe.  The exp-then-quantize
// kernel is the exception: there two lanes share a block (see its section
// below).
//
// Rules: "Online MXFP6" page ("Start a model": packed codes and an E8M0
// scale per 32 values); "EFQ-Softmax" explainer (exponent-only block scale
// from the largest magnitude inside the block; exp-then-quantize); "AXS-6" page
// ("Overview" block layout; "Quick Start" fused fake-quantize).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_exp.h"
#include "mx_formats.h"
#include "mx_hw.h"
#include "mx_kernels.h"

namespace mxk {

constexpr uint32_t kNaN32 = 0x7FC00000u;
constexpr uint32_t kNaN16x2 = 0x7FC07FC0u;

// ---------------------------------------------------------------------------
// Memory helpers: block b of a 16-bit tensor (bf16 or fp16) is 4 x 16 B at
// b*64, of fp32 8 x 16 B at b*128; packed codes are W dwords at b*4W.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_block16(const void* x, int64_t b, uint32_t (&d)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(x) + b * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = p[i];
    d[4 * i] = q.x; d[4 * i + 1] = q.y; d[4 * i + 2] = q.z; d[4 * i + 3] = q.w;
  }
}

__device__ __forceinline__ void load_f32_block(const void* x, int64_t b, uint32_t (&d)[32]) {
  const uint4* p = reinterpret_cast<const uint4*>(x) + b * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 q = p[i];
    d[4 * i] = q.x; d[4 * i + 1] = q.y; d[4 * i + 2] = q.z; d[4 * i + 3] = q.w;
  }
}

template <int N>
__device__ __forceinline__ void store_dwords16(void* y, int64_t b, const uint32_t (&d)[N]) {
  static_assert(N % 4 == 0, "whole 16-byte chunks");
  uint4* p = reinterpret_cast<uint4*>(y) + b * (N / 4);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) p[i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
}

template <int W>
__device__ __forceinline__ void store_codes(void* codes, int64_t b, const uint32_t (&o)[W]) {
  if constexpr (W == 6) {
    uint2* p = reinterpret_cast<uint2*>(codes) + b * 3;
    p[0] = make_uint2(o[0], o[1]);
    p[1] = make_uint2(o[2], o[3]);
    p[2] = make_uint2(o[4], o[5]);
  } else {
    store_dwords16<W>(codes, b, o);
  }
}

template <int W>
__device__ __forceinline__ void load_codes(const void* codes, int64_t b, uint32_t (&o)[W]) {
  if constexpr (W == 6) {
    const uint2* p = reinterpret_cast<const uint2*>(codes) + b * 3;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 q = p[i];
      o[2 * i] = q.x;
      o[2 * i + 1] = q.y;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(codes) + b * (W / 4);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 q = p[i];
      o[4 * i] = q.x; o[4 * i + 1] = q.y; o[4 * i + 2] = q.z; o[4 * i + 3] = q.w;
    }
  }
}

// Canonical NaN for every NaN value (fp32 patterns / packed bf16 pairs).
__device__ __forceinline__ uint32_t canon_nan32(uint32_t u) {
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? kNaN32 : u;
}
__device__ __forceinline__ uint32_t canon_nan16x2(uint32_t u) {
  const uint32_t lo = (u & 0x7FFFu) > 0x7F80u ? 0x7FC0u : (u & 0xFFFFu);
  const uint32_t hi = ((u >> 16) & 0x7FFFu) > 0x7F80u ? 0x7FC0u : (u >> 16);
  return lo | (hi << 16);
}

// ---------------------------------------------------------------------------
// Wide per-block outputs (64 B of bf16 or 128 B of fp32 per lane) go through
// LDS: lane l writes its block's NCH 16-byte chunks into row l of a padded
// per-wave tile (row pitch NCH+1 chunks, so the 16 lanes of one LDS pass hit
// distinct banks), then the wave writes the tile back chunk-major, so that
// every store instruction covers 64 consecutive chunks (1 KB) of HBM.
// Writing lane-strided 16-byte pieces directly costs ~45 % more time on the
// write-heavy decoders.  Only chunks of blocks below nb are stored.
// ---------------------------------------------------------------------------
constexpr int kTile = 64;  // blocks per wave tile (one per lane)

template <int NCH>
__device__ __forceinline__ void store_tile_via_lds_full(uint4* __restrict__ lds, void* y,
                                                        int64_t b0, int64_t nb, int lane,
                                                        const uint32_t (&d)[4 * NCH]) {
  constexpr int P = NCH + 1;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    lds[lane * P + i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t valid = (nb - b0 < kTile ? nb - b0 : kTile) * NCH;  // chunks to store
  uint4* dst = reinterpret_cast<uint4*>(y) + b0 * NCH;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * kTile + lane;  // chunk index within the tile
    if (c < valid) dst[c] = lds[(c / NCH) * P + (c % NCH)];
  }
  // the next tile's writes into lds must follow these reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The same for 128-byte (fp32) blocks in two rounds of 32 lanes, through a
// tile half the size (32 rows of NCH+1 chunks), so that a workgroup needs
// 18 KB of LDS instead of 37 KB and twice as many fit on a CU: lanes 0..31
// park their blocks and the wave stores them (4 KB, four 1 KB
// instructions), then lanes 32..63 do the same.
template <int NCH>
__device__ __forceinline__ void store_tile_via_lds_halves(uint4* __restrict__ lds, void* y,
                                                          int64_t b0, int64_t nb, int lane,
                                                          const uint32_t (&d)[4 * NCH]) {
  constexpr int P = NCH + 1;
  constexpr int HALF = kTile / 2;  // blocks per round
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((lane >> 5) == half) {
      const int row = lane & (HALF - 1);
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        lds[row * P + i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t hb0 = b0 + half * HALF;
    const int64_t left = nb - hb0;
    const int64_t valid = (left < 0 ? 0 : (left < HALF ? left : HALF)) * NCH;
    uint4* dst = reinterpret_cast<uint4*>(y) + hb0 * NCH;
#pragma unroll
    for (int i = 0; i < HALF * NCH / 64; ++i) {
      const int c = i * 64 + lane;
      if (c < valid) dst[c] = lds[(c / NCH) * P + (c % NCH)];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// LDS slots per wave for a tile of NCH-chunk blocks, and the store that
// uses them: fp32 blocks (NCH = 8) go out in two rounds through half a
// tile (measured: the fp32 E2M1 dequantizer of the attention probabilities
// 454 -> 438 us), bf16 blocks in one.
constexpr int tile_slots(int nch) { return (nch == 8 ? kTile / 2 : kTile) * (nch + 1); }

template <int NCH>
__device__ __forceinline__ void store_tile_via_lds(uint4* __restrict__ lds, void* y, int64_t b0,
                                                   int64_t nb, int lane,
                                                   const uint32_t (&d)[4 * NCH]) {
  if constexpr (NCH == 8) store_tile_via_lds_halves<NCH>(lds, y, b0, nb, lane, d);
  else store_tile_via_lds_full<NCH>(lds, y, b0, nb, lane, d);
}

// ---------------------------------------------------------------------------
// Tensor element types, as the C ABI's mx_dtype.  fp16 tensors (the "Online
// MXFP6" page, "Start a model": BF16 or FP16 weights) have bf16's 64-byte
// blocks.  The MX encoders take fp16 values directly (the fp16-source
// scaled conversions); AXS-6 and eXmY widen them to fp32 in registers
// (exactly) and take the fp32 paths.  fp16 outputs are fp32 results rounded
// once to binary16 (nearest even, overflow to infinity; the canonical fp32
// NaN becomes 0x7E00).
// ---------------------------------------------------------------------------
constexpr int kBF16 = 0, kF32 = 1, kF16 = 2;

// 16-byte output chunks per block of a tensor of type dt
constexpr int out_chunks(int dt) { return dt == kF32 ? 8 : 4; }

__device__ __forceinline__ uint32_t f16_to_f32_bits(uint32_t h) {
  return __float_as_uint((float)__builtin_bit_cast(_Float16, (uint16_t)h));
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(uint32_t f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(f));
}

// 32 fp16 values (16 dwords, element 2k in the low half of dword k) as
// fp32 patterns; exact.
__device__ __forceinline__ void widen_f16(const uint32_t (&d)[16], uint32_t (&v)[32]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    v[2 * k] = f16_to_f32_bits(d[k] & 0xFFFFu);
    v[2 * k + 1] = f16_to_f32_bits(d[k] >> 16);
  }
}

// The 32 values of block b as fp32 patterns, from an fp32 or fp16 tensor.
template <int DT>
__device__ __forceinline__ void load_wide(const void* x, int64_t b, uint32_t (&v)[32]) {
  if constexpr (DT == kF16) {
    uint32_t d[16];
    load_block16(x, b, d);
    widen_f16(d, v);
  } else {
    load_f32_block(x, b, v);
  }
}

// A lane's 32 fp32 results stored through the wave's LDS tile into an fp32
// or fp16 tensor.
template <int DT>
__device__ __forceinline__ void store_wide(uint4* __restrict__ lds, void* y, int64_t b0,
                                           int64_t nb, int lane, const uint32_t (&out)[32]) {
  if constexpr (DT == kF16) {
    uint32_t h[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      h[k] = f32_to_f16_bits(out[2 * k]) | (f32_to_f16_bits(out[2 * k + 1]) << 16);
    store_tile_via_lds<4>(lds, y, b0, nb, lane, h);
  } else {
    store_tile_via_lds<8>(lds, y, b0, nb, lane, out);
  }
}

// ---------------------------------------------------------------------------
// Coalesced input for a wave tile of 64 blocks of 16-bit values (4 KB of
// bf16 or fp16): four direct
// global->LDS loads, each covering 1 KB of consecutive bytes, then lane l
// reads its block's four 16-byte quarters from LDS.  The quarters of block
// b sit at slots 4b + (q ^ ((b / 4) % 4)): the 16 lanes of one LDS read
// cycle (blocks 16c..16c+15, one quarter each) then hit 16 distinct slots,
// and the map is its own inverse, so lane l of load i fetches the piece that
// slot 64i + l holds.  tile (wave-uniform) must hold 256 slots; it is free
// for other use once the function returns (every lane has its block in
// registers).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glob_void_t;

__device__ __forceinline__ int quarter_slot(int b, int q) { return 4 * b + (q ^ ((b >> 2) & 3)); }

__device__ __forceinline__ void load_tile16_coalesced(const void* x, int64_t b0, uint4* tile,
                                                         int lane, uint32_t (&d)[16]) {
  const uint4* src = reinterpret_cast<const uint4*>(x) + 4 * b0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int S = 64 * i + lane;
    __builtin_amdgcn_global_load_lds((glob_void_t*)(src + quarter_slot(S >> 2, S & 3)),
                                     (lds_void_t*)(tile + 64 * i), 16, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = tile[quarter_slot(lane, q)];
    d[4 * q] = v.x; d[4 * q + 1] = v.y; d[4 * q + 2] = v.z; d[4 * q + 3] = v.w;
  }
  // the caller's stores reuse the tile region only after every lane has
  // read its block
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave tile t of a 16-bit tensor of nb blocks: lane l gets block 64 t + l,
// read through LDS in 1 KB instructions when the tile is whole (the MX
// quantizer reads its input this way 1.5-3.4 % faster than with four
// 16-byte loads per lane), else directly; fn(b, d) runs for each block
// b < nb.  t is the same for the whole wave.
template <typename Fn>
__device__ __forceinline__ void wave_tile16(const void* x, int64_t t, int64_t nb, uint4* tile,
                                               int lane, Fn&& fn) {
  const int64_t b0 = t * kTile, b = b0 + lane;
  uint32_t d[16] = {};
  if (b0 + kTile <= nb) load_tile16_coalesced(x, b0, tile, lane, d);
  else if (b < nb) load_block16(x, b, d);
  if (b < nb) fn(b, d);
}

// ---------------------------------------------------------------------------
// MX formats (E2M3, E3M2, E2M1, E4M3): hardware conversions
// ---------------------------------------------------------------------------
// Block b of one tensor from its values of type DT (16 dwords of bf16 or
// fp16 pairs, or 32 fp32 patterns): scale byte, codes, and both stores.
template <int F, int DT>
__device__ __forceinline__ void quantize_mx_values(const uint32_t (&d)[DT == kF32 ? 32 : 16],
                                                   int64_t b, void* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  constexpr int W = Fmt<F>::W;
  uint32_t o[W];
  uint32_t byte;
  if constexpr (DT == kBF16) {
    byte = scale_byte_from_amax<F>(amax_bf16x32(d));
    encode_bf16<F>(d, scale_operand(byte), o);
  } else if constexpr (DT == kF16) {
    byte = scale_byte_from_amax<F>(amax_f16x32(d));
    encode_f16<F>(d, scale_operand(byte), o);
  } else {
    byte = scale_byte_from_amax<F>(amax_f32x32(d));
    encode_f32<F>(d, scale_operand(byte), o);
  }
  if (byte == 0xFFu) {
#pragma unroll
    for (int k = 0; k < W; ++k) o[k] = 0u;
  }
  store_codes<W>(codes, b, o);
  scales[b] = (uint8_t)byte;
}

// bf16 and fp16 input: one wave tile of 64 blocks per wave (wave_tile16);
// fp32 input: one block per lane.
template <int F, int DT>
__global__ __launch_bounds__(256) void quantize_mx(const void* __restrict__ x, int64_t nb,
                                                   void* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  if constexpr (DT != kF32) {
    __shared__ uint4 lds[4][4 * kTile];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves)
      wave_tile16(x, t, nb, lds[wave], lane, [&](int64_t b, const uint32_t (&d)[16]) {
        quantize_mx_values<F, DT>(d, b, codes, scales);
      });
  } else {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
      uint32_t d[32];
      load_wide<DT>(x, b, d);
      quantize_mx_values<F, DT>(d, b, codes, scales);
    }
  }
}

// Several tensors in one launch: workgroup w belongs to the tensor i with
// wg_start[i] <= w < wg_start[i + 1] (found from blockIdx and the kernel
// arguments alone, so i is uniform and its pointers are scalar loads), and
// its lanes take blocks 256 (w - wg_start[i]) + lane of that tensor.
template <int F, int DT>
__global__ __launch_bounds__(256) void quantize_mx_batch(const QuantBatch a) {
  const uint32_t w = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 1; k < kBatchMax; ++k) i = (k < a.n && w >= a.wg_start[k]) ? k : i;
  // one block per lane with direct loads: the wave-tile loads of
  // quantize_mx measured no faster on the conversion's layer batches
  const int64_t b = (int64_t)(w - a.wg_start[i]) * 256 + threadIdx.x;
  if (b < a.nb[i]) {
    if constexpr (DT != kF32) {
      uint32_t d[16];
      load_block16(a.x[i], b, d);
      quantize_mx_values<F, DT>(d, b, a.codes[i], a.scales[i]);
    } else {
      uint32_t d[32];
      load_wide<DT>(a.x[i], b, d);
      quantize_mx_values<F, DT>(d, b, a.codes[i], a.scales[i]);
    }
  }
}

template <int F, int DT>
__global__ __launch_bounds__(256) void dequantize_mx(const void* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     int64_t nb, void* __restrict__ y) {
  constexpr int W = Fmt<F>::W;
  constexpr int NCH = out_chunks(DT);  // 16-byte output chunks per block
  __shared__ uint4 lds[4][tile_slots(NCH)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves) {
    const int64_t b0 = t * kTile, b = b0 + lane;
    uint32_t o[W] = {};
    uint32_t byte = 0;
    if (b < nb) {
      load_codes<W>(codes, b, o);
      byte = scales[b];
    }
    bool fix_nan = (byte == 0xFFu);
    if constexpr (F == F_E4M3) fix_nan |= e4m3_has_nan_code(o);
    if constexpr (DT == kBF16) {
      uint32_t d[16];
      decode_bf16<F>(o, scale_operand(byte), d);
      if (fix_nan) {
#pragma unroll
        for (int k = 0; k < 16; ++k) d[k] = (byte == 0xFFu) ? kNaN16x2 : canon_nan16x2(d[k]);
      }
      store_tile_via_lds<4>(lds[wave], y, b0, nb, lane, d);
    } else {
      uint32_t d[32];
      decode_f32<F>(o, scale_operand(byte), d);
      if (fix_nan) {
#pragma unroll
        for (int k = 0; k < 32; ++k) d[k] = (byte == 0xFFu) ? kNaN32 : canon_nan32(d[k]);
      }
      store_wide<DT>(lds[wave], y, b0, nb, lane, d);
    }
  }
}

template <int F, int DT>
__global__ __launch_bounds__(256) void fake_quantize_mx(const void* x, int64_t nb, void* y) {
  constexpr int W = Fmt<F>::W;
  constexpr int NCH = out_chunks(DT);
  __shared__ uint4 lds[4][tile_slots(NCH)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves) {
    const int64_t b0 = t * kTile, b = b0 + lane;
    uint32_t o[W];
    uint32_t d[DT == kBF16 ? 16 : 32] = {};
    if constexpr (DT == kBF16) {
      if (b0 + kTile <= nb) load_tile16_coalesced(x, b0, lds[wave], lane, d);  // whole tile
      else if (b < nb) load_block16(x, b, d);
      const uint32_t byte = scale_byte_from_amax<F>(amax_bf16x32(d));
      const float sc = scale_operand(byte);
      encode_bf16<F>(d, sc, o);
      decode_bf16<F>(o, sc, d);
      if (byte == 0xFFu) {
#pragma unroll
        for (int k = 0; k < 16; ++k) d[k] = kNaN16x2;
      }
    } else {
      uint32_t byte;
      if constexpr (DT == kF16) {  // encoded from the fp16 values, decoded to fp32
        uint32_t h[16] = {};
        if (b0 + kTile <= nb) load_tile16_coalesced(x, b0, lds[wave], lane, h);  // whole tile
        else if (b < nb) load_block16(x, b, h);
        byte = scale_byte_from_amax<F>(amax_f16x32(h));
        encode_f16<F>(h, scale_operand(byte), o);
      } else {
        if (b < nb) load_wide<DT>(x, b, d);
        byte = scale_byte_from_amax<F>(amax_f32x32(d));
        encode_f32<F>(d, scale_operand(byte), o);
      }
      const float sc = scale_operand(byte);
      decode_f32<F>(o, sc, d);
      if (byte == 0xFFu) {
#pragma unroll
        for (int k = 0; k < 32; ++k) d[k] = kNaN32;
      }
    }
    // every lane has read its block before any lane of the wave stores, so
    // y == x is safe
    if constexpr (DT == kBF16) store_tile_via_lds<4>(lds[wave], y, b0, nb, lane, d);
    else store_wide<DT>(lds[wave], y, b0, nb, lane, d);
  }
}

// ---------------------------------------------------------------------------
// AXS-6: sign + 5-bit magnitude m, value m/16 under the shared exponent.
// m = min(rint(|v| * 2^(131 - byte)), 31) in fp32 (exact scaling; RNE).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t axs6_block_byte(const uint32_t (&v)[32]) {
  uint32_t amax = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = max(amax, v[k] & 0x7FFFFFFFu);
  return scale_byte_from_amax<F_AXS6>(amax);
}

template <int DT>
__device__ __forceinline__ void load_values(const void* x, int64_t b, uint32_t (&v)[32]) {
  if constexpr (DT == kBF16) {
    uint32_t d[16];
    load_block16(x, b, d);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[2 * k] = d[k] << 16;
      v[2 * k + 1] = d[k] & 0xFFFF0000u;
    }
  } else {
    load_wide<DT>(x, b, v);
  }
}

// Block b from its 32 values (fp32 patterns) and its byte.
__device__ __forceinline__ void quantize_axs6_values(const uint32_t (&v)[32], uint32_t byte,
                                                     int64_t b, void* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     uint8_t* __restrict__ aux) {
  uint32_t c[32], o[6];
  // m = min(rint(16 |v| / X), 31) with 16 |v| / X = |v| 2^(131 - byte)
  // exactly (as in fake_quantize_axs6); the sign bit is v's
  const int e_in = 131 - (int)byte;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float m = __builtin_fminf(
        __builtin_rintf(__builtin_ldexpf(__builtin_fabsf(__uint_as_float(v[k])), e_in)), 31.0f);
    c[k] = (uint32_t)m | ((v[k] >> 26) & 32u);
  }
  pack32<6>(c, o);
  if (byte == 0xFFu) {  // rare: a block with a NaN or an infinity has no codes
#pragma unroll
    for (int k = 0; k < 6; ++k) o[k] = 0u;
  }
  store_codes<6>(codes, b, o);
  scales[b] = (uint8_t)byte;
  // config plane: 2 bits per block, all zero (the uniform grid)
  if ((b & 3) == 0) aux[b >> 2] = 0;
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_axs6(const void* __restrict__ x, int64_t nb,
                                                     void* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     uint8_t* __restrict__ aux) {
  // one block per lane with direct loads: on the 32 MB AXS-6 weight the
  // wave-tile loads of the other quantizers measured 2.6 % slower
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    uint32_t v[32];
    uint32_t byte;
    if constexpr (DT == kBF16) {
      uint32_t d[16];
      load_block16(x, b, d);
      byte = scale_byte_from_amax<F_AXS6>(amax_bf16x32(d));
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[2 * k] = d[k] << 16;
        v[2 * k + 1] = d[k] & 0xFFFF0000u;
      }
    } else {
      load_values<DT>(x, b, v);
      byte = axs6_block_byte(v);
    }
    quantize_axs6_values(v, byte, b, codes, scales, aux);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void fake_quantize_axs6(const void* x, int64_t nb, void* y) {
  constexpr int NCH = out_chunks(DT);
  __shared__ uint4 lds[4][tile_slots(NCH)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves) {
    const int64_t b0 = t * kTile, b = b0 + lane;
    uint32_t v[32] = {};
    uint32_t byte;
    if constexpr (DT == kBF16) {
      uint32_t d[16] = {};
      if (b0 + kTile <= nb) load_tile16_coalesced(x, b0, lds[wave], lane, d);  // whole tile
      else if (b < nb) load_block16(x, b, d);
      byte = scale_byte_from_amax<F_AXS6>(amax_bf16x32(d));
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[2 * k] = d[k] << 16;
        v[2 * k + 1] = d[k] & 0xFFFF0000u;
      }
    } else {
      if constexpr (DT == kF16) {
        uint32_t h[16] = {};
        if (b0 + kTile <= nb) load_tile16_coalesced(x, b0, lds[wave], lane, h);  // whole tile
        else if (b < nb) load_block16(x, b, h);
        widen_f16(h, v);
      } else if (b < nb) {
        load_values<DT>(x, b, v);
      }
      byte = axs6_block_byte(v);
    }
    // the same rounding as quantize_axs6, on signed values: 16 |v| / X =
    // |v| 2^(131 - byte) exactly (a value small enough to lose bits there
    // rounds to zero either way), rint is symmetric (so a negative value
    // that rounds to zero gives -0), and clamping the rounded value to
    // [-31, 31] equals clamping |v| / X to 31/16 first; the result
    // m 2^(byte - 131) is exact
    const int e_in = 131 - (int)byte, e_out = (int)byte - 131;
    uint32_t out[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float m = __builtin_amdgcn_fmed3f(
          __builtin_rintf(__builtin_ldexpf(__uint_as_float(v[k]), e_in)), -31.0f, 31.0f);
      out[k] = __float_as_uint(__builtin_ldexpf(m, e_out));
    }
    const bool poisoned = byte == 0xFFu;  // a block with a NaN or an infinity
    if constexpr (DT == kBF16) {
      // every result is a bf16 value: keep the top halves
      uint32_t d[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        d[k] = poisoned ? kNaN16x2 : __builtin_amdgcn_perm(out[2 * k + 1], out[2 * k], 0x07060302u);
      store_tile_via_lds<4>(lds[wave], y, b0, nb, lane, d);
    } else {
#pragma unroll
      for (int k = 0; k < 32; ++k) out[k] = poisoned ? kNaN32 : out[k];
      store_wide<DT>(lds[wave], y, b0, nb, lane, out);
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void dequantize_axs6(const void* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const uint8_t* __restrict__ aux, int64_t nb,
                                                       void* __restrict__ y) {
  constexpr int NCH = out_chunks(DT);
  __shared__ uint4 lds[4][tile_slots(NCH)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves) {
    const int64_t b0 = t * kTile, b = b0 + lane;
    uint32_t o[6] = {};
    uint32_t byte = 0;
    bool poisoned = false;
    if (b < nb) {
      load_codes<6>(codes, b, o);
      byte = scales[b];
      poisoned = (byte == 0xFFu) || (((aux[b >> 2] >> (2 * (b & 3))) & 3u) != 0u);
    }
    const int sexp = (int)byte - 127;
    uint32_t out[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t code = unpack1<6>(o, k);
      const float val = decode_mag<F_AXS6>(code & 31u, sexp);
      out[k] = poisoned ? kNaN32 : (__float_as_uint(val) | ((code >> 5) << 31));
    }
    if constexpr (DT == kBF16) {
      uint32_t d[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        d[k] = f32_to_bf16_rne(__uint_as_float(out[2 * k])) |
               (f32_to_bf16_rne(__uint_as_float(out[2 * k + 1])) << 16);
      store_tile_via_lds<4>(lds[wave], y, b0, nb, lane, d);
    } else {
      store_wide<DT>(lds[wave], y, b0, nb, lane, out);
    }
  }
}

// ---------------------------------------------------------------------------
// Generic eXmY formats (the eXmY abstract: any split of a bit width into
// exponent and mantissa bits): no hardware conversion exists for most of
// them, so rounding is done in fp32.  W (3..9 bits) is a template parameter;
// the split comes in ExmyParams.
// Rounding of a scaled, clamped magnitude a (exact in fp32): the grid step
// at a is 2^(max(floor(log2 a), emin) - m).  Adding C = 2^(that exponent +
// 23) makes the fp32 adder's round-to-nearest-even land on that step (the
// sum lies in [C, 2C), whose ulp is the step), so n = bits(a + C) - bits(C)
// counts steps and mag = n + (binade - emin) << m.  Ties then go to the
// even n, which is the even code whenever m >= 1; with m = 0 (exponent only)
// a tie 1.5 * 2^k would pick the larger value, so an odd code there is
// moved down by one.
// ---------------------------------------------------------------------------
template <bool M0>
__device__ __forceinline__ uint32_t exmy_round(float a, const ExmyParams& p) {
  // a >= 0, at most the largest magnitude.  eb = max(a's biased exponent,
  // 127 + emin) - (127 + emin), one saturating subtraction: which of the
  // format's binades holds a (0 also below 2^emin, where the codes are
  // subnormal).  The grid step at a is 2^(eb + emin - m); adding C =
  // 2^(eb + emin + 23 - m) leaves a rounded to that step (nearest, ties to
  // even) as the sum's mantissa field (the sum lies in [C, 2C)), and the
  // binade's first code is eb << m.  C's exponent field is eb plus a
  // constant of the format, kept in a scalar register.
  const uint32_t ab = __float_as_uint(a);
  const uint32_t emin_b = (uint32_t)(127 + p.emin);
  const uint32_t eb = __builtin_elementwise_sub_sat(ab >> 23, emin_b);
  const uint32_t c0 = __builtin_amdgcn_readfirstlane((emin_b + (uint32_t)(23 - p.m)) << 23);
  const float C = __uint_as_float((eb << 23) + c0);
  uint32_t mag = (__float_as_uint(a + C) & 0x7FFFFFu) + (eb << p.m);
  if constexpr (M0) {
    // exponent-only formats: a tie between two powers of two goes to the
    // even exponent field, which the adder does not know about
    if ((ab >> 23) >= emin_b && (ab & 0x7FFFFFu) == 0x400000u && (mag & 1u)) mag -= 1u;
  }
  return mag;
}

// e8m0 (exponent only: zero and 2^-126 .. 2^128).  A block's top binade of
// scaled values, [2^128, 2^129), lies beyond fp32, so its codes come from h =
// a / 2 = |v| 2^(126 - byte), clamped to 2^127 (p.maxf).  The scaling is
// exact: a finite block has byte <= 126, so it never shifts a bit out.
// Magnitude code k >= 1 is h = 2^(k - 128).  A normal h = 2^(F - 127) (1 +
// M 2^-23) lies between codes F + 1 and F + 2, its midpoint at M = 2^22 going
// to the even code; an fp32-subnormal h is compared with the midpoints 2^-128
// (codes 0 and 1) and 1.5 2^-127 (codes 1 and 2), ties to the even code.
__device__ __forceinline__ uint32_t e8m0_code_of_half(float h) {
  const uint32_t b = __float_as_uint(h), F = b >> 23, M = b & 0x7FFFFFu;
  const uint32_t up = (M > 0x400000u) | ((M == 0x400000u) & ((F + 1u) & 1u));
  const uint32_t sub = M <= 0x200000u ? 0u : (M < 0x600000u ? 1u : 2u);
  return F ? F + 1u + up : sub;
}

// e8m0's magnitude code k times 2^scale_exp: 2^(k - 127 + scale_exp), rounded
// by ldexp (to inf above fp32, to a subnormal or zero below it); code 0 is 0.
__device__ __forceinline__ float e8m0_decode(uint32_t mag, int scale_exp) {
  return mag ? __builtin_ldexpf(1.0f, (int)mag - 127 + scale_exp) : 0.0f;
}

__device__ __forceinline__ uint32_t exmy_byte_from_amax(uint32_t amax, const ExmyParams& p) {
  if (amax >= 0x7F800000u) return 0xFFu;
  if (amax == 0u) return 0u;
  const int field = (int)(amax >> 23);
  const int e = field ? field - 127 : (31 - __builtin_clz(amax)) - 149;
  int b = e - p.emax + 127;
  b = b < 0 ? 0 : b;
  return (uint32_t)(b > 254 ? 254 : b);
}

// The value of magnitude code mag times 2^scale_exp (exact before the
// final rounding of ldexp).  Normal codes: the fp32 bit pattern is mag
// shifted so its exponent field lands on fp32's, plus the bias difference.
// Subnormal codes (exponent field 0, and every code of an integer format):
// the same pattern reads (1 + mant / 2^m) 2^-bias, and 2x - 2^(1 - bias)
// is mant / 2^m 2^(1 - bias).
__device__ __forceinline__ float exmy_decode(uint32_t mag, int scale_exp, const ExmyParams& p) {
  const float f = __uint_as_float((mag << (23 - p.m)) + p.dec_bits);
  const float sub = __builtin_fmaf(f, 2.0f, p.dec_sub);
  return __builtin_ldexpf(mag < (1u << p.m) ? sub : f, scale_exp);
}

__device__ __forceinline__ uint32_t exmy_block_byte(const uint32_t (&v)[32], const ExmyParams& p) {
  return exmy_byte_from_amax(amax_f32x32(v), p);
}

template <int W, bool M0>
__device__ __forceinline__ void exmy_codes(const uint32_t (&v)[32], uint32_t byte,
                                           const ExmyParams& p, uint32_t (&c)[32]) {
  // a poisoned block (byte 0xFF) gives arbitrary codes here; the callers
  // zero them
  if constexpr (W == 9 && M0) {  // e8m0
    const int sh = 126 - (int)byte;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float h = fminf(__builtin_ldexpf(__builtin_fabsf(__uint_as_float(v[k])), sh), p.maxf);
      c[k] = e8m0_code_of_half(h) | ((v[k] >> 31) << 8);
    }
    return;
  }
  const int neg_exp = 127 - (int)byte;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float a =
        fminf(__builtin_ldexpf(__builtin_fabsf(__uint_as_float(v[k])), neg_exp), p.maxf);
    c[k] = exmy_round<M0>(a, p) | ((v[k] >> 31) << (W - 1));
  }
}

// The value of a magnitude code times 2^scale_exp, for any split.
template <bool E8>
__device__ __forceinline__ float exmy_value(uint32_t mag, int scale_exp, const ExmyParams& p) {
  if constexpr (E8) return e8m0_decode(mag, scale_exp);
  return exmy_decode(mag, scale_exp, p);
}

template <int W, int DT, bool M0>
__global__ __launch_bounds__(256) void quantize_exmy(const void* __restrict__ x, int64_t nb,
                                                     uint32_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, ExmyParams p) {
  auto block = [&](int64_t b, const uint32_t (&v)[32], uint32_t byte) {
    uint32_t c[32], o[W];
    exmy_codes<W, M0>(v, byte, p, c);
    pack32<W>(c, o);
#pragma unroll
    for (int j = 0; j < W; ++j) codes[b * W + j] = byte == 0xFFu ? 0u : o[j];  // 4W bytes
    scales[b] = (uint8_t)byte;
  };
  if constexpr (DT != kF32) {
    // bf16 and fp16 input: one wave tile of 64 blocks per wave (wave_tile16)
    __shared__ uint4 lds[4][4 * kTile];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves)
      wave_tile16(x, t, nb, lds[wave], lane, [&](int64_t b, const uint32_t (&d)[16]) {
        uint32_t v[32];
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            v[2 * k] = d[k] << 16;
            v[2 * k + 1] = d[k] & 0xFFFF0000u;
          }
          block(b, v, exmy_byte_from_amax(amax_bf16x32(d), p));
        } else {
          widen_f16(d, v);
          block(b, v, exmy_byte_from_amax(amax_f16x32(d), p));
        }
      });
  } else {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
      uint32_t v[32];
      load_wide<DT>(x, b, v);
      block(b, v, exmy_byte_from_amax(amax_f32x32(v), p));
    }
  }
}

template <int W, int DT, bool M0>
__global__ __launch_bounds__(256) void fake_quantize_exmy(const void* x, int64_t nb, void* y,
                                                          ExmyParams p) {
  constexpr int NCH = out_chunks(DT);
  __shared__ uint4 lds[4][tile_slots(NCH)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves) {
    const int64_t b0 = t * kTile, b = b0 + lane;
    uint32_t v[32] = {}, c[32], out[32];
    if (b < nb) load_values<DT>(x, b, v);
    const uint32_t byte = exmy_block_byte(v, p);
    exmy_codes<W, M0>(v, byte, p, c);
    const int sexp = (int)byte - 127;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float val = exmy_value<W == 9 && M0>(c[k] & ((1u << (W - 1)) - 1u), sexp, p);
      out[k] = (byte == 0xFFu) ? kNaN32 : (__float_as_uint(val) | (v[k] & 0x80000000u));
    }
    if constexpr (DT == kBF16) {
      // the results are bf16 values: round to nearest even (exact unless a
      // subnormal product needs it)
      uint32_t d[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        d[k] = f32_to_bf16_rne(__uint_as_float(out[2 * k])) |
               (f32_to_bf16_rne(__uint_as_float(out[2 * k + 1])) << 16);
      store_tile_via_lds<4>(lds[wave], y, b0, nb, lane, d);
    } else {
      store_wide<DT>(lds[wave], y, b0, nb, lane, out);
    }
  }
}

template <int W, int DT, bool E8>
__global__ __launch_bounds__(256) void dequantize_exmy(const uint32_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       int64_t nb, void* __restrict__ y,
                                                       ExmyParams p) {
  constexpr int NCH = out_chunks(DT);
  __shared__ uint4 lds[4][tile_slots(NCH)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t * kTile < nb; t += nwaves) {
    const int64_t b0 = t * kTile, b = b0 + lane;
    uint32_t o[W] = {};
    uint32_t byte = 0;
    if (b < nb) {
#pragma unroll
      for (int j = 0; j < W; ++j) o[j] = codes[b * W + j];
      byte = scales[b];
    }
    const int sexp = (int)byte - 127;
    uint32_t out[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t code = unpack1<W>(o, k);
      const float val = exmy_value<E8>(code & ((1u << (W - 1)) - 1u), sexp, p);
      out[k] = __float_as_uint(val) | ((code >> (W - 1)) << 31);
    }
    if (byte == 0xFFu) {  // rare: a poisoned block
#pragma unroll
      for (int k = 0; k < 32; ++k) out[k] = kNaN32;
    }
    if constexpr (DT == kBF16) {
      // every eXmY value has at most 8 significant bits, so it is a bf16
      // value whenever it is an fp32 normal (or zero, inf, NaN): the top
      // half of the bit pattern, no rounding.  Only blocks whose smallest
      // nonzero magnitude is an fp32 subnormal take the rounding path.
      uint32_t d[16];
      if (p.emin - p.m + sexp >= -126 || byte == 0xFFu) {
#pragma unroll
        for (int k = 0; k < 16; ++k) d[k] = __builtin_amdgcn_perm(out[2 * k + 1], out[2 * k], 0x07060302u);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          d[k] = f32_to_bf16_rne(__uint_as_float(out[2 * k])) |
                 (f32_to_bf16_rne(__uint_as_float(out[2 * k + 1])) << 16);
      }
      store_tile_via_lds<4>(lds[wave], y, b0, nb, lane, d);
    } else {
      store_wide<DT>(lds[wave], y, b0, nb, lane, out);
    }
  }
}

// ---------------------------------------------------------------------------
// Exp-then-quantize probabilities: one wavefront per row (exp_ref_nonpos is
// the fixed fp32 exp sequence, in mx_exp.h).  Two lanes share a block: lanes
// 2i and 2i+1 hold its two 16-value halves, so a lane reads 64 contiguous
// bytes per half block (fp32 rows stream ~25 % faster that way on this part
// than with a whole 128-byte block per lane), and the pair exchanges its
// half maxima with one DPP move before deriving the block's scale.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Largest of the wave's 64 values (NaN-free inputs), in every lane: DPP
// within each row of 16 lanes (swap pairs, swap pair-of-pairs, mirror the
// half row, mirror the row), then the four row results read as scalars.
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, dpp_f32<0xB1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp_f32<0x4E>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_f32<0x140>(m));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// max of v over lanes 2i and 2i+1 (DPP quad_perm [1,0,3,2] swaps the pair)
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ void load_f32_half(const float* row, int64_t h, uint32_t (&d)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(row) + 4 * h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = p[i];
    d[4 * i] = q.x; d[4 * i + 1] = q.y; d[4 * i + 2] = q.z; d[4 * i + 3] = q.w;
  }
}

// Half block hg (global index) of packed codes: W2 dwords at hg * 4 * W2.
template <int W2>
__device__ __forceinline__ void store_half(void* codes, int64_t hg, const uint32_t (&o)[W2]) {
  if constexpr (W2 == 2) {
    reinterpret_cast<uint2*>(codes)[hg] = make_uint2(o[0], o[1]);
  } else if constexpr (W2 == 4) {
    reinterpret_cast<uint4*>(codes)[hg] = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    static_assert(W2 == 3, "FP6 half blocks are 3 dwords");
    uint32_t* p = reinterpret_cast<uint32_t*>(codes) + 3 * hg;
    p[0] = o[0]; p[1] = o[1]; p[2] = o[2];
  }
}

// Probabilities of one half block of shifted scores and its codes under the
// block's scale; `kind` is the row's case: 0 finite row max, 1 row max +inf
// (then s - m is -inf, giving P = 0, except NaN where s is +inf itself).
// Every lane of the wave calls it together (the pair exchange).
template <int F>
__device__ __forceinline__ void probs_half(const uint32_t (&sv)[16], float m, int kind,
                                           uint32_t (&o)[Fmt<F>::W / 2], uint32_t& byte) {
  uint32_t v[16];
  if (kind == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = __float_as_uint(exp_ref_nonpos(__uint_as_float(sv[k]) - m));
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = (sv[k] == 0x7F800000u) ? 0x7FC00000u : 0u;
  }
  uint32_t amax = 0u;  // P >= 0 (or NaN), so the bit patterns order as values
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = max(amax, v[k]);
  byte = scale_byte_from_amax<F>(pair_max(amax));
  encode_f32_half<F>(v, scale_operand(byte), o);
  if (byte == 0xFFu) {
#pragma unroll
    for (int k = 0; k < Fmt<F>::W / 2; ++k) o[k] = 0u;
  }
}

// One wavefront per row of nh = 2 * cols / 32 half blocks (the launcher
// splits row counts beyond one grid).  HB > 0: lane l
// keeps half blocks l, l+64, ... (at most HB of them, enough for the whole
// row) in registers, so the row is read once.  HB == 0: rows of any length;
// the second pass reads the row again.  Half blocks past the row's end read
// nothing (their values are -inf, so P = 0) and store nothing; the two
// halves of a block are always on the same side of the end.  FULL: nh is
// exactly 64 * HB, so no lane needs that test (exec-masked loads and stores
// cost ~4 % of the kernel's time on 4096-column rows).
// Occupancy: five waves per SIMD where the row fits (the kernel streams
// reads and writes at once, and four waves leave the memory system short of
// requests), two for rows of 512 half blocks (128 registers of row data).
template <int F, int HB, bool FULL>
__global__ __launch_bounds__(256, HB == 8 ? 2 : 5) void softmax_quantize_rows(const float* __restrict__ s,
                                                             int64_t rows, int64_t cols,
                                                             void* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  constexpr int W2 = Fmt<F>::W / 2;
  constexpr uint32_t kNegInf = 0xFF800000u;
  const int lane = threadIdx.x & 63;
  const int64_t nbr = cols >> 5, nh = 2 * nbr;
  {
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= rows) return;
    // per-row bases are the same for the whole wave; lane offsets are small
    const float* srow = s + row * cols;
    uint8_t* crow = reinterpret_cast<uint8_t*>(codes) + row * nh * (4 * W2);
    uint8_t* srow_scales = scales + row * nbr;
    uint32_t keep[HB > 0 ? HB : 1][16];
    // pass 1: exact row maximum; a NaN anywhere poisons the whole row
    float m = -__builtin_inff();
    bool nan_seen = false;
    if constexpr (HB > 0) {
      // every load of the row is issued before the first use, so the whole
      // row is in flight at once
#pragma unroll
      for (int i = 0; i < HB; ++i) {
        if (FULL || lane + 64 * i < nh) {
          load_f32_half(srow, lane + 64 * i, keep[i]);
        } else {
#pragma unroll
          for (int k = 0; k < 16; ++k) keep[i][k] = kNegInf;
        }
      }
#pragma unroll
      for (int i = 0; i < HB; ++i) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float x = __uint_as_float(keep[i][k]);
          nan_seen |= (x != x);
          m = fmaxf(m, x);
        }
      }
    } else {
      for (int64_t h = lane; h < nh; h += 64) {
        uint32_t v[16];
        load_f32_half(srow, h, v);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float x = __uint_as_float(v[k]);
          nan_seen |= (x != x);
          m = fmaxf(m, x);
        }
      }
    }
    m = wave_max(m);
    // a NaN in the row, or a row of only -inf (then s - m = -inf - -inf is
    // NaN everywhere), poisons every block of the row
    const bool row_nan = __ballot(nan_seen) != 0 || m == -__builtin_inff();
    const int kind = (m == __builtin_inff()) ? 1 : 0;
    // pass 2: P = exp(s - m) per half block, then the block's scale and codes
    if constexpr (HB > 0) {
#pragma unroll
      for (int i = 0; i < HB; ++i) {
        const int h = lane + 64 * i;
        uint32_t o[W2];
        uint32_t byte = 0xFFu;
        if (row_nan) {
#pragma unroll
          for (int k = 0; k < W2; ++k) o[k] = 0u;
        } else {
          probs_half<F>(keep[i], m, kind, o, byte);
        }
        if (FULL || h < nh) {
          store_half<W2>(crow, h, o);
          if (!(lane & 1)) srow_scales[h >> 1] = (uint8_t)byte;
        }
      }
    } else {
      // the loop bound is the same for every lane, so whole pairs take part
      for (int64_t h0 = 0; h0 < nh; h0 += 64) {
        const int64_t h = h0 + lane;
        uint32_t o[W2];
        uint32_t byte = 0xFFu;
        if (row_nan) {
#pragma unroll
          for (int k = 0; k < W2; ++k) o[k] = 0u;
        } else {
          uint32_t sv[16];
          if (h < nh) {
            load_f32_half(srow, h, sv);
          } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) sv[k] = kNegInf;
          }
          probs_half<F>(sv, m, kind, o, byte);
        }
        if (h < nh) {
          store_half<W2>(crow, h, o);
          if (!(lane & 1)) srow_scales[h >> 1] = (uint8_t)byte;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline dim3 grid_for(int64_t work, int per_wg) {
  int64_t g = (work + per_wg - 1) / per_wg;
  if (g > 0x7FFFFFFF) g = 0x7FFFFFFF;
  if (g < 1) g = 1;
  return dim3((unsigned)g);
}

#define MXK_SWITCH_MX(fmt, BODY)                                   \
  switch (fmt) {                                                   \
    case F_E2M3: { constexpr int FF = F_E2M3; BODY; } break;       \
    case F_E3M2: { constexpr int FF = F_E3M2; BODY; } break;       \
    case F_E2M1: { constexpr int FF = F_E2M1; BODY; } break;       \
    case F_E4M3: { constexpr int FF = F_E4M3; BODY; } break;       \
    default: return hipErrorInvalidValue;                          \
  }

#define MXK_SWITCH_DT(dt, BODY)                                  \
  switch (dt) {                                                  \
    case kBF16: { constexpr int DD = kBF16; BODY; } break;       \
    case kF32: { constexpr int DD = kF32; BODY; } break;         \
    case kF16: { constexpr int DD = kF16; BODY; } break;         \
    default: return hipErrorInvalidValue;                        \
  }

hipError_t launch_quantize(int fmt, int dt, const void* x, int64_t nb, void* codes,
                           uint8_t* scales, uint8_t* aux, hipStream_t st) {
  const dim3 grid = grid_for(nb, 256), block(256);
  if (fmt == F_AXS6) {
    MXK_SWITCH_DT(dt, hipLaunchKernelGGL(quantize_axs6<DD>, grid, block, 0, st, x, nb, codes,
                                         scales, aux));
    return hipGetLastError();
  }
  MXK_SWITCH_MX(fmt, MXK_SWITCH_DT(dt, hipLaunchKernelGGL((quantize_mx<FF, DD>), grid, block, 0,
                                                           st, x, nb, codes, scales)));
  return hipGetLastError();
}

hipError_t launch_quantize_batch(int fmt, int dt, const QuantBatch& a, hipStream_t st) {
  if (a.n < 1 || a.n > kBatchMax) return hipErrorInvalidValue;
  const dim3 grid(a.wg_start[a.n]), block(256);
  MXK_SWITCH_MX(fmt, MXK_SWITCH_DT(dt, hipLaunchKernelGGL((quantize_mx_batch<FF, DD>), grid,
                                                           block, 0, st, a)));
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, int dt, const void* codes, const uint8_t* scales,
                             const uint8_t* aux, int64_t nb, void* y, hipStream_t st) {
  const dim3 grid = grid_for(nb, 4 * kTile), block(256);  // one 64-block tile per wave
  if (fmt == F_AXS6) {
    MXK_SWITCH_DT(dt, hipLaunchKernelGGL(dequantize_axs6<DD>, grid, block, 0, st, codes, scales,
                                         aux, nb, y));
    return hipGetLastError();
  }
  MXK_SWITCH_MX(fmt, MXK_SWITCH_DT(dt, hipLaunchKernelGGL((dequantize_mx<FF, DD>), grid, block, 0,
                                                           st, codes, scales, nb, y)));
  return hipGetLastError();
}

hipError_t launch_fake_quantize(int fmt, int dt, const void* x, int64_t nb, void* y,
                                hipStream_t st) {
  const dim3 grid = grid_for(nb, 4 * kTile), block(256);  // one 64-block tile per wave
  if (fmt == F_AXS6) {
    MXK_SWITCH_DT(dt, hipLaunchKernelGGL(fake_quantize_axs6<DD>, grid, block, 0, st, x, nb, y));
    return hipGetLastError();
  }
  MXK_SWITCH_MX(fmt, MXK_SWITCH_DT(dt, hipLaunchKernelGGL((fake_quantize_mx<FF, DD>), grid, block,
                                                           0, st, x, nb, y)));
  return hipGetLastError();
}

// Rows that fill HB half blocks per lane exactly take the variant without
// end-of-row tests.
template <int F, int HB>
static void launch_rows(dim3 grid, hipStream_t st, const float* s, int64_t rows, int64_t cols,
                        void* codes, uint8_t* scales) {
  if constexpr (HB > 0) {
    if (2 * (cols / 32) == 64 * HB) {
      hipLaunchKernelGGL((softmax_quantize_rows<F, HB, true>), grid, dim3(256), 0, st, s, rows,
                         cols, codes, scales);
      return;
    }
  }
  hipLaunchKernelGGL((softmax_quantize_rows<F, HB, false>), grid, dim3(256), 0, st, s, rows, cols,
                     codes, scales);
}

hipError_t launch_softmax_quantize(int fmt, const float* s, int64_t rows, int64_t cols,
                                   void* codes, uint8_t* scales, hipStream_t st) {
  const int64_t nbr = cols / 32, nh = 2 * nbr;
  // one wave per row, four per workgroup; a grid holds 2^31 - 1 workgroups
  const int64_t kRowsPerLaunch = 4 * (int64_t)0x7FFFFFFF;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t n = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const dim3 grid = grid_for(n, 4);
    const float* sp = s + r0 * cols;
    uint8_t* sc = scales + r0 * nbr;
    void* cp = nullptr;
    // rows of up to 64, 128, 256 or 512 half blocks stay in registers (read once)
    MXK_SWITCH_MX(fmt, {
      cp = static_cast<uint8_t*>(codes) + r0 * nbr * (4 * Fmt<FF>::W);
      if (nh <= 64)
        (launch_rows<FF, 1>)(grid, st, sp, n, cols, cp, sc);
      else if (nh <= 128)
        (launch_rows<FF, 2>)(grid, st, sp, n, cols, cp, sc);
      else if (nh <= 256)
        (launch_rows<FF, 4>)(grid, st, sp, n, cols, cp, sc);
      else if (nh <= 512)
        (launch_rows<FF, 8>)(grid, st, sp, n, cols, cp, sc);
      else
        (launch_rows<FF, 0>)(grid, st, sp, n, cols, cp, sc);
    });
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

#define MXK_SWITCH_WIDTH(w, BODY)                           \
  switch (w) {                                              \
    case 3: { constexpr int WW = 3; BODY; } break;          \
    case 4: { constexpr int WW = 4; BODY; } break;          \
    case 5: { constexpr int WW = 5; BODY; } break;          \
    case 6: { constexpr int WW = 6; BODY; } break;          \
    case 7: { constexpr int WW = 7; BODY; } break;          \
    case 8: { constexpr int WW = 8; BODY; } break;          \
    case 9: { constexpr int WW = 9; BODY; } break;          \
    default: return hipErrorInvalidValue;                   \
  }

hipError_t launch_exmy(int op, int width, const ExmyParams& p, int dt, const void* in,
                       const uint8_t* scales_in, int64_t nb, void* out, uint8_t* scales_out,
                       hipStream_t st) {
  const dim3 block(256);
  const dim3 grid = (op == 0) ? grid_for(nb, 256) : grid_for(nb, 4 * kTile);
  // exponent-only formats (m = 0) need the even-exponent tie rule; width 9
  // with m = 0 is e8m0, which has code paths of its own
#define MXK_EXMY_LAUNCH(M0)                                                                    \
  MXK_SWITCH_WIDTH(width, MXK_SWITCH_DT(dt, {                                                  \
    if (op == 0)                                                                               \
      hipLaunchKernelGGL((quantize_exmy<WW, DD, M0>), grid, block, 0, st, in, nb,              \
                         (uint32_t*)out, scales_out, p);                                       \
    else if (op == 1)                                                                          \
      hipLaunchKernelGGL((dequantize_exmy<WW, DD, M0 && WW == 9>), grid, block, 0, st,         \
                         (const uint32_t*)in, scales_in, nb, out, p);                          \
    else                                                                                       \
      hipLaunchKernelGGL((fake_quantize_exmy<WW, DD, M0>), grid, block, 0, st, in, nb, out, p); \
  }))
  if (p.m == 0) {
    MXK_EXMY_LAUNCH(true);
  } else {
    MXK_EXMY_LAUNCH(false);
  }
#undef MXK_EXMY_LAUNCH
  return hipGetLastError();
}

}  // namespace mxk
