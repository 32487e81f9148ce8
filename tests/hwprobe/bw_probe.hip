// bw_probe.hip -- the HBM ceiling of the bf16 -> FP6 quantizer's byte mix.
//
// Copy kernels that move the quantizer's bytes in several access schedules
// with no arithmetic beyond folding every input word into the outputs, so
// that the compiler keeps every load; the first (mix_copy) has one lane per
// 32-value block doing four 16-byte loads of its 64 bf16 bytes, three
// 8-byte stores of 24 "code" bytes and one scale byte.  The benchmark times
// them beside the quantizer on the same buffers; this is measurement
// infrastructure, not part of the library.
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

// ---------------------------------------------------------------------------
// Other access schedules for the same byte mix (64 bytes read, 24 + 1
// written per 32-value block), to find the fastest one this HBM allows:
//   variant 0  one lane per block with direct 16-byte loads (mix_copy above)
//   variant 1  the same, with workgroups renumbered so that each of the 8
//              XCDs (which receive consecutive workgroups in turn) covers
//              one contiguous eighth of the tensor
//   variant 2  4 blocks per lane, all 16 loads of a lane issued before any
//              store; the workgroup's 1024 blocks then leave as one
//              contiguous 24 KB run of codes (staged in LDS) and 1 KB of
//              scales
//   variant 3  variant 2 with the XCD renumbering
//   variant 4  read only (the same loads as variant 0, one dword written
//              per workgroup), the read half of the mix
//   variant 5  write only (the same stores as variant 0, nothing read),
//              the write half of the mix
//   variants 6, 7, 8  variant 0 with device-scope (sc1), nontemporal (nt)
//              and system-scope (sc0 sc1) stores
//   variants 9, 10, 11  writes only, reads only, and the whole mix, with
//              every instruction of a wave covering 1 KB of consecutive
//              bytes (whole workgroups of 256 blocks only)
//   variant 12 the bf16 MX quantizer's schedule: a wave's 64 blocks (4 KB)
//              reach LDS by four direct global->LDS loads of 1 KB each,
//              then every lane reads its block from LDS and stores like
//              variant 0 (whole waves only)
//   variant 13 the loads of variant 12 alone (one dword written per wave)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t xcd_order(int64_t wg, int64_t total) {
  return (total & 7) == 0 ? (wg & 7) * (total >> 3) + (wg >> 3) : wg;
}

// Store cache policies: 0 the default; 1 device scope (relaxed atomic
// stores at agent scope, which carry the sc1 bit: written through the
// XCD's L2); 2 nontemporal (the nt bit); 3 system scope (sc0 sc1).
template <int POL>
__device__ __forceinline__ void store_u64(uint64_t* p, uint64_t v) {
  if constexpr (POL == 0) *p = v;
  else if constexpr (POL == 1) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else if constexpr (POL == 2) __builtin_nontemporal_store(v, p);
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <int POL>
__device__ __forceinline__ void store_u8(uint8_t* p, uint8_t v) {
  if constexpr (POL == 0) *p = v;
  else if constexpr (POL == 1) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else if constexpr (POL == 2) __builtin_nontemporal_store(v, p);
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <bool XCD, int POL = 0>
__global__ __launch_bounds__(256) void mix_copy_grid(const uint4* __restrict__ x, int64_t nb,
                                                     uint64_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t wg = XCD ? xcd_order(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t b = wg * 256 + threadIdx.x;
  if (b >= nb) return;
  const uint4 q0 = x[4 * b], q1 = x[4 * b + 1], q2 = x[4 * b + 2], q3 = x[4 * b + 3];
  const uint32_t o0 = q0.x ^ q2.z, o1 = q0.y ^ q2.w, o2 = q0.z ^ q3.x, o3 = q0.w ^ q3.y;
  const uint32_t o4 = q1.x ^ q1.z ^ q3.z, o5 = q1.y ^ q1.w ^ q3.w ^ q2.x ^ q2.y;
  store_u64<POL>(codes + 3 * b, o0 | ((uint64_t)o1 << 32));
  store_u64<POL>(codes + 3 * b + 1, o2 | ((uint64_t)o3 << 32));
  store_u64<POL>(codes + 3 * b + 2, o4 | ((uint64_t)o5 << 32));
  store_u8<POL>(scales + b, (uint8_t)(o0 ^ o5));
}

template <bool XCD>
__global__ __launch_bounds__(256) void mix_copy_phase(const uint4* __restrict__ x, int64_t nb,
                                                      uint4* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  constexpr int C = 4;  // blocks per lane
  __shared__ uint32_t lds[256 * C * 6];
  const int t = threadIdx.x;
  const int64_t wg = XCD ? xcd_order(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t b0 = wg * 256 * C;
  uint4 q[C][4];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int64_t b = b0 + 256 * c + t;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[c][i] = b < nb ? x[4 * b + i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int lb = 256 * c + t;  // block within the workgroup's chunk
    uint32_t* o = lds + 6 * lb;
    o[0] = q[c][0].x ^ q[c][2].z; o[1] = q[c][0].y ^ q[c][2].w; o[2] = q[c][0].z ^ q[c][3].x;
    o[3] = q[c][0].w ^ q[c][3].y; o[4] = q[c][1].x ^ q[c][1].z ^ q[c][3].z;
    o[5] = q[c][1].y ^ q[c][1].w ^ q[c][3].w ^ q[c][2].x ^ q[c][2].y;
    const int64_t b = b0 + lb;
    if (b < nb) scales[b] = (uint8_t)(o[0] ^ o[5]);
  }
  __syncthreads();
  // the chunk's codes: 256 * C * 24 bytes = 384 * C 16-byte pieces
  const int64_t valid = (nb - b0 < 256 * C ? nb - b0 : 256 * C) * 24 / 16;  // whole pieces
  const uint4* l4 = reinterpret_cast<const uint4*>(lds);
#pragma unroll
  for (int i = 0; i < (384 * C) / 256; ++i) {
    const int p = 256 * i + t;
    if (p < valid) codes[b0 * 24 / 16 + p] = l4[p];
  }
}

__global__ __launch_bounds__(256) void mix_read_only(const uint4* __restrict__ x, int64_t nb,
                                                     uint32_t* __restrict__ sink) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  if (b < nb) {
    const uint4 q0 = x[4 * b], q1 = x[4 * b + 1], q2 = x[4 * b + 2], q3 = x[4 * b + 3];
    acc = q0.x ^ q0.y ^ q0.z ^ q0.w ^ q1.x ^ q1.y ^ q1.z ^ q1.w ^ q2.x ^ q2.y ^ q2.z ^ q2.w ^
          q3.x ^ q3.y ^ q3.z ^ q3.w;
  }
  // a store that depends on every loaded word keeps every load alive; it
  // happens only for one value, so almost nothing is written
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void mix_write_only(int64_t nb, uint2* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  const uint32_t v = (uint32_t)b * 2654435761u;
  codes[3 * b] = make_uint2(v, v + 1);
  codes[3 * b + 1] = make_uint2(v + 2, v + 3);
  codes[3 * b + 2] = make_uint2(v + 4, v + 5);
  scales[b] = (uint8_t)v;
}

// Fully coalesced forms: every load or store instruction of a wave covers
// 64 consecutive 16-byte pieces (1 KB).  A workgroup's 256 blocks are 1024
// input pieces, 384 code pieces and 16 scale pieces.
template <bool READ, bool WRITE>
__global__ __launch_bounds__(256) void mix_coalesced(const uint4* __restrict__ x, int64_t nb,
                                                     uint4* __restrict__ codes,
                                                     uint4* __restrict__ scales,
                                                     uint32_t* __restrict__ sink) {
  const int t = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * 256;
  if (b0 + 256 > nb) return;  // whole workgroups only (timing probe)
  uint4 q[4] = {};
  if constexpr (READ) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = x[4 * b0 + 256 * i + t];
  }
  uint4 o0 = make_uint4(q[0].x ^ q[2].z, q[0].y ^ q[2].w, q[0].z ^ q[3].x, q[0].w ^ q[3].y);
  uint4 o1 = make_uint4(q[1].x ^ q[1].z, q[1].y ^ q[1].w, q[3].z ^ q[2].x, q[3].w ^ q[2].y);
  if constexpr (!READ) {
    o0 = make_uint4(t, t + 1, t + 2, t + 3);
    o1 = make_uint4(t + 4, t + 5, t + 6, t + 7);
  }
  if constexpr (WRITE) {
    uint4* c = codes + b0 * 24 / 16;
    c[t] = o0;
    if (t < 128) c[256 + t] = o1;
    if (t < 16) scales[b0 / 16 + t] = make_uint4(o0.x ^ o1.y, o0.y, o0.z, o0.w ^ o1.x);
  } else {
    const uint32_t acc = o0.x ^ o0.y ^ o0.z ^ o0.w ^ o1.x ^ o1.y ^ o1.z ^ o1.w;
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glob_void_t;

// 16-byte quarter q of tile block b sits in LDS slot 4b + (q ^ ((b / 4) % 4)),
// so the 16 lanes of one LDS read cycle hit 16 distinct slots; the map is
// its own inverse, so lane l of load i fetches the piece slot 64 i + l holds
__device__ __forceinline__ int tile_slot(int b, int q) { return 4 * b + (q ^ ((b >> 2) & 3)); }

template <bool WRITE>
__global__ __launch_bounds__(256) void mix_lds_loads(const uint4* __restrict__ x, int64_t nb,
                                                     uint64_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     uint32_t* __restrict__ sink) {
  __shared__ uint4 tile[4][256];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (b0 + 64 > nb) return;  // whole waves only (timing probe)
  const uint4* src = x + 4 * b0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int S = 64 * i + lane;
    __builtin_amdgcn_global_load_lds((glob_void_t*)(src + tile_slot(S >> 2, S & 3)),
                                     (lds_void_t*)(&tile[wave][64 * i]), 16, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint4 q0 = tile[wave][tile_slot(lane, 0)], q1 = tile[wave][tile_slot(lane, 1)];
  const uint4 q2 = tile[wave][tile_slot(lane, 2)], q3 = tile[wave][tile_slot(lane, 3)];
  const int64_t b = b0 + lane;
  const uint32_t o0 = q0.x ^ q2.z, o1 = q0.y ^ q2.w, o2 = q0.z ^ q3.x, o3 = q0.w ^ q3.y;
  const uint32_t o4 = q1.x ^ q1.z ^ q3.z, o5 = q1.y ^ q1.w ^ q3.w ^ q2.x ^ q2.y;
  if constexpr (WRITE) {
    codes[3 * b] = o0 | ((uint64_t)o1 << 32);
    codes[3 * b + 1] = o2 | ((uint64_t)o3 << 32);
    codes[3 * b + 2] = o4 | ((uint64_t)o5 << 32);
    scales[b] = (uint8_t)(o0 ^ o5);
  } else {
    // a store that depends on every loaded word keeps every load alive
    const uint32_t acc = o0 ^ o1 ^ o2 ^ o3 ^ o4 ^ o5 ^ q0.x ^ q2.x ^ q2.y;
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
  }
}

// variant as above; x: nb * 64 bytes, codes: nb * 24 bytes (16-byte
// aligned), scales: nb bytes, sink: at least ceil(nb / 256) dwords (variants
// 4, 10 and 13).  Returns hipGetLastError(), or -1 for an unknown variant.
extern "C" int probe_mix_variant(int variant, const void* x, int64_t nb, void* codes,
                                 uint8_t* scales, uint32_t* sink, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nb < 1) return -1;
  const int64_t g1 = (nb + 255) / 256;          // one block per lane
  const int64_t g4 = (nb + 1023) / 1024;        // four blocks per lane
  const int64_t g1x = (g1 + 7) / 8 * 8;         // padded to whole XCD rounds
  const int64_t g4x = (g4 + 7) / 8 * 8;
  if (g1x > 0x7FFFFFFF) return -1;
  const uint4* xi = static_cast<const uint4*>(x);
  switch (variant) {
    case 0: return probe_mix_copy(x, nb, codes, scales, stream);
    case 1:
      hipLaunchKernelGGL((mix_copy_grid<true, 0>), dim3((unsigned)g1x), dim3(256), 0, st, xi, nb,
                         static_cast<uint64_t*>(codes), scales);
      break;
    case 6:
      hipLaunchKernelGGL((mix_copy_grid<false, 1>), dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint64_t*>(codes), scales);
      break;
    case 7:
      hipLaunchKernelGGL((mix_copy_grid<false, 2>), dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint64_t*>(codes), scales);
      break;
    case 8:
      hipLaunchKernelGGL((mix_copy_grid<false, 3>), dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint64_t*>(codes), scales);
      break;
    case 2:
      hipLaunchKernelGGL(mix_copy_phase<false>, dim3((unsigned)g4), dim3(256), 0, st, xi, nb,
                         static_cast<uint4*>(codes), scales);
      break;
    case 3:
      hipLaunchKernelGGL(mix_copy_phase<true>, dim3((unsigned)g4x), dim3(256), 0, st, xi, nb,
                         static_cast<uint4*>(codes), scales);
      break;
    case 4:
      hipLaunchKernelGGL(mix_read_only, dim3((unsigned)g1), dim3(256), 0, st, xi, nb, sink);
      break;
    case 5:
      hipLaunchKernelGGL(mix_write_only, dim3((unsigned)g1), dim3(256), 0, st, nb,
                         static_cast<uint2*>(codes), scales);
      break;
    case 9:
      hipLaunchKernelGGL((mix_coalesced<false, true>), dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint4*>(codes), reinterpret_cast<uint4*>(scales), sink);
      break;
    case 10:
      hipLaunchKernelGGL((mix_coalesced<true, false>), dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint4*>(codes), reinterpret_cast<uint4*>(scales), sink);
      break;
    case 11:
      hipLaunchKernelGGL((mix_coalesced<true, true>), dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint4*>(codes), reinterpret_cast<uint4*>(scales), sink);
      break;
    case 12:
      hipLaunchKernelGGL(mix_lds_loads<true>, dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint64_t*>(codes), scales, sink);
      break;
    case 13:
      hipLaunchKernelGGL(mix_lds_loads<false>, dim3((unsigned)g1), dim3(256), 0, st, xi, nb,
                         static_cast<uint64_t*>(codes), scales, sink);
      break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// A copy of arbitrary byte counts per 32-value block, for the floor of any
// kernel's byte mix: workgroup w reads its 256 blocks' in_bpb bytes each
// (one contiguous run of 256 in_bpb bytes) and writes 256 out_bpb bytes,
// every instruction covering 16 bytes per lane of consecutive memory; every
// loaded word is folded into the stored ones, so the stores wait for all
// of the workgroup's loads, as in the kernels.  in_bpb and out_bpb must be
// multiples of 1/16 of a block's bytes such that 256 in_bpb and 256 out_bpb
// are multiples of 16 (always true for whole bytes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bytes_copy(const uint4* __restrict__ x, int64_t in_pieces,
                                                  uint4* __restrict__ y, int64_t out_pieces,
                                                  int wg_in, int wg_out) {
  const int t = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int64_t i0 = w * wg_in, o0 = w * wg_out;
  uint4 acc = make_uint4(t, 0, 0, 0);
  for (int p = t; p < wg_in; p += 256) {
    if (i0 + p < in_pieces) {
      const uint4 v = x[i0 + p];
      acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
    }
  }
  for (int p = t; p < wg_out; p += 256) {
    if (o0 + p < out_pieces) y[o0 + p] = make_uint4(acc.x + p, acc.y, acc.z, acc.w);
  }
}

// x: nb * in_bpb bytes, y: nb * out_bpb bytes (rounded up to 16-byte
// pieces; device memory, 16-byte aligned).  -1 for a bad size.
extern "C" int probe_bytes_copy(const void* x, int64_t nb, int in_bpb, void* y, int out_bpb,
                                void* stream) {
  if (nb < 1 || in_bpb < 1 || out_bpb < 1 || (256 * in_bpb) % 16 || (256 * out_bpb) % 16) return -1;
  const int64_t g = (nb + 255) / 256;
  if (g > 0x7FFFFFFF) return -1;
  const int64_t in_pieces = (nb * in_bpb + 15) / 16, out_pieces = (nb * out_bpb + 15) / 16;
  hipLaunchKernelGGL(bytes_copy, dim3((unsigned)g), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(x), in_pieces, static_cast<uint4*>(y), out_pieces,
                     256 * in_bpb / 16, 256 * out_bpb / 16);
  return (int)hipGetLastError();
}
