// mx_attention.hip -- attention forward with exp-then-quantize E2M1
// probabilities on gfx950 (device code and its launcher).
//
// Method: the EFQ-Softmax explainer, sections "Does it change
// FlashAttention?" and the stage table: the online softmax keeps a running
// row maximum, rescales the earlier sums when it grows, accumulates in wide
// registers and divides once; the probabilities are exp() of the shifted
// scores, quantized to block-scaled E2M1 (MXFP4) for the PV product, and
// the same E2M1 block is summed for the normalizer.
//
// Work split: one workgroup of 4 waves per (head, 128 queries); each wave
// owns 32 queries and walks the keys in tiles of 64:
//   S^T  = K_tile * Q^T      8+8 bf16 32x32x16 MFMAs whose A rows are the
//                            tile's keys in a permuted order, chosen so that
//                            each lane receives the 32 scores of one
//                            (query, 32-key block) pair with no exchange
//   t    = S * c with c = scale * log2(e) (scores in powers of two); tile
//          max; rescale O and l when the maximum grows
//   p    = 2^(t - m) (exp2_ref); block scale byte; 16 E2M1 codes per lane,
//          which are exactly the lane's B operand of the block-scaled MFMA
//          (EFQ: codes from one fused multiply-add per raw score instead)
//   O^T += V^T * P^T         4 block-scaled 32x32x64 MFMAs (V in E4M3,
//                            E2M3, E3M2 or E2M1, P in E2M1)
//   l   += 1 * P^T           one more block-scaled MFMA with an all-ones A
// so the probabilities never leave registers and the PV product and the
// normalizing sum consume the same E2M1 operand.  K and V^T tiles are
// staged in LDS once per workgroup and shared by its 4 waves.
//
// Operand layouts (checked on the hardware by the library's probe tests):
//   bf16 32x32x16: lane l holds A[l%32][8(l/32) + e] and B[8(l/32) + e][l%32]
//   scaled 32x32x64, FP6/FP4: lane l holds the 32-value block k = 32(l/32)..
//     of row (A) or column (B) l%32; FP8: bytes 0..15 hold k = 16(l/32) + e
//     and bytes 16..31 hold k = 32 + 16(l/32) + e; the lane's scale operand
//     is the E8M0 of block k = 32(l/32).. of that row or column
//   result: D[8(r/4) + 4(l/32) + r%4][l%32] in accumulator r.
// The head-dimension index inside the QK^T contraction is permuted (lane
// half h, step i, element e -> d = 64h + 8i + e) so that every lane reads
// 128 contiguous bytes of its Q and K rows; the sum is the same.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mx_exp2.h"
#include "mx_formats.h"
#include "mx_hw.h"
#include "mx_kernels.h"

namespace mxk {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glob_void_t;

constexpr int kD = 128;              // head dimension
constexpr int kTile = 64;            // keys per online-softmax step
constexpr int kWaves = 4;           // waves per workgroup (a multiple of 4)
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;   // queries per workgroup
constexpr int kKBytes = kTile * 2 * kD;  // one K tile in LDS: 64 rows of 256 B

// Score layout.  The two 32x32 score MFMAs of a tile give lane (col, h) the
// output rows rho = 8g + 4h + e (g = 0..3, e = 0..3) of column col.  The
// first MFMA's A row rho holds key 32h + 8g + e of the tile and the
// second's key 32h + 8g + 4 + e, so lane half h ends up with exactly the
// keys of the tile's block h: accumulator r of the first MFMA is key
// 8(r/4) + r%4 of the block and of the second key 8(r/4) + 4 + r%4.  A lane
// therefore reads K row kperm(col) = 32((col/4) % 2) + 8(col/8) + col%4 for
// the first MFMA and kperm(col) + 4 for the second.
__device__ __forceinline__ int kperm(int col) {
  return 32 * ((col >> 2) & 1) + 8 * (col >> 3) + (col & 3);
}

// LDS layouts.  Tiles arrive by direct global->LDS loads, where lane i of
// a wave writes the 16-byte slot i of a contiguous run (a 12-byte load
// fills the first 12 bytes of its slot), so conflict-free reads come from
// XOR-swizzling the slot order inside a row instead of padding.
//   K: row r (key), 16-B chunk L (8 values of one row) in slot L ^ kswz(r),
//      kswz(r) = r%4 + 4((r/32) % 2) + 8((r/8) % 2): the 16 lanes of one
//      LDS read cycle (columns 16c..16c+15) read rows kperm(col) (+ 4),
//      whose kswz is col % 16, so they hit 16 distinct slots.
//   V^T, two blocks of row d: E4M3 4 chunks of 16 B, E2M3/E3M2 4 chunks of
//      12 B (half a block each), chunk L in slot L ^ ((d / 2) % 4); E2M1 2
//      chunks of 16 B, chunk L in slot L ^ ((d / 4) % 2).
template <int VF> struct VTile;
template <> struct VTile<0> {
  static constexpr int BPB = 32, CH = 16, CPR = 4;
  __device__ static int swz(int d) { return (d >> 1) & 3; }
};
__device__ __forceinline__ int kswz(int r) {
  return (r & 3) | (((r >> 5) & 1) << 2) | (((r >> 3) & 1) << 3);
}
template <> struct VTile<2> {
  static constexpr int BPB = 24, CH = 12, CPR = 4;
  __device__ static int swz(int d) { return (d >> 1) & 3; }
};
template <> struct VTile<3> : VTile<2> {};
template <> struct VTile<4> {
  static constexpr int BPB = 16, CH = 16, CPR = 2;
  __device__ static int swz(int d) { return (d >> 2) & 1; }
};

// The A operand (V^T row d = 32T + col, lane half h) of the block-scaled
// MFMA from the LDS copy of the tile's two blocks of that row.  The swizzle
// of row d depends only on col, so a lane's two chunk offsets inside row
// col (v_offsets) serve every T; rows 32T + col are 32T rows further on,
// which the LDS reads take as immediate offsets.
template <int VF>
__device__ __forceinline__ void v_offsets(int col, int h, uint32_t& lo, uint32_t& hi) {
  using L = VTile<VF>;
  const int z = L::swz(col);
  const int base = col * L::CPR * 16;
  if constexpr (VF == 0) {
    lo = (uint32_t)(base + 16 * (h ^ z));
    hi = (uint32_t)(base + 16 * ((2 + h) ^ z));
  } else if constexpr (VF == 4) {
    lo = hi = (uint32_t)(base + 16 * (h ^ z));
  } else {
    lo = (uint32_t)(base + 16 * ((2 * h) ^ z));
    hi = (uint32_t)(base + 16 * ((2 * h + 1) ^ z));
  }
}

template <int VF>
__device__ __forceinline__ i32x8_t load_v_operand(const uint8_t* vt, int T, uint32_t lo_off,
                                                  uint32_t hi_off) {
  using L = VTile<VF>;
  const uint8_t* rows = vt + T * 32 * L::CPR * 16;
  i32x8_t a = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (VF == 0) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(rows + lo_off);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(rows + hi_off);
    a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
    a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
  } else if constexpr (VF == 4) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(rows + lo_off);
    a[0] = w[0]; a[1] = w[1]; a[2] = w[2]; a[3] = w[3];
  } else {
    const u32x3_t lo = *reinterpret_cast<const u32x3_t*>(rows + lo_off);
    const u32x3_t hi = *reinterpret_cast<const u32x3_t*>(rows + hi_off);
    a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = hi[0]; a[4] = hi[1]; a[5] = hi[2];
  }
  return a;
}

// One direct global->LDS load: lane i of the wave writes its 16 (12) bytes
// at l + 16 i (12 i); l must be the same for the whole wave.
__device__ __forceinline__ void lds_load16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((glob_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
__device__ __forceinline__ void lds_load12(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((glob_void_t*)g, (lds_void_t*)l, 12, 0, 0);
}

// Direct loads of one key tile into one LDS buffer.  Each wave issues
// 16 / kWaves K and up to 8 / kWaves V instructions; every lane's address is a fixed per-lane
// offset plus a per-tile base that is the same for the whole wave, so the
// per-tile cost is scalar arithmetic.  K rows past lk and a missing second
// V block (a last tile of 32 keys) re-read valid data; the kernel masks
// their products.
template <int VF>
struct TileLoader {
  using L = VTile<VF>;
  const uint8_t* kh;  // this head's K
  const uint8_t* vh;  // this head's V^T codes
  int64_t vstep;      // bytes of the V^T rows one round of instructions covers
  uint32_t koff[2];   // lane's K byte offset inside a tile (instruction 0; rows 0..31, 32..63)
  uint32_t voff;      // lane's V byte offset (instruction 0, tile 0)
  uint32_t vhalf;     // bytes back to the first block when the lane's chunk is in the second
  int lk, nbk, wave;

  __device__ void init(const uint16_t* k, const uint8_t* vc, int bh, int lk_, int nbk_,
                       int wave_, int lane) {
    lk = lk_;
    nbk = nbk_;
    wave = wave_;
    kh = reinterpret_cast<const uint8_t*>(k) + (int64_t)bh * lk * (2 * kD);
    vh = vc + (int64_t)bh * kD * nbk * L::BPB;
    vstep = (int64_t)(kThreads / L::CPR) * nbk * L::BPB;
    // K chunk c = 64 (4 n + wave) + lane: row 16 n + 4 wave + lane / 16,
    // slot lane % 16, logical chunk slot ^ kswz(row); kswz changes with n
    // only through row bit 5 (n >= 2)
    static_assert(kWaves == 4, "the K swizzle offsets assume 16 rows per round");
    const int r0 = 4 * wave + (lane >> 4);
    koff[0] = (uint32_t)(r0 * 256 + 16 * ((lane & 15) ^ kswz(r0)));
    koff[1] = (uint32_t)(r0 * 256 + 16 * ((lane & 15) ^ kswz(r0 + 32)));
    // V chunk c = 64 (kWaves n + wave) + lane: row c / CPR, slot c % CPR (n
    // adds kThreads / CPR rows and does not change the swizzle)
    const int c0 = wave * 64 + lane;
    const int d0 = c0 / L::CPR;
    const int ch = (c0 - d0 * L::CPR) ^ L::swz(d0);
    voff = (uint32_t)(d0 * nbk * L::BPB + L::CH * ch);
    vhalf = ch >= L::CPR / 2 ? (uint32_t)(L::CH * (L::CPR / 2)) : 0u;
  }

  __device__ __forceinline__ void issue(uint8_t* ksb, uint8_t* vsb, int jt) const {
    const int key0 = jt * kTile, kb0 = 2 * jt;
    const bool two = kb0 + 1 < nbk;
    const uint8_t* kt = kh + (int64_t)key0 * (2 * kD);
    constexpr int kRowsPerRound = 4 * kWaves;
#pragma unroll
    for (int n = 0; n < kTile / kRowsPerRound; ++n) {
      // rows 32.. of a 32-key last tile do not exist: re-read rows 0..
      const int r = n * kRowsPerRound;
      const uint8_t* base = kt + (int64_t)(r - ((!two && r >= 32) ? 32 : 0)) * (2 * kD);
      lds_load16(base + koff[n >= 2], ksb + (kWaves * n + wave) * 64 * 16);
    }
    const uint32_t vo = two ? voff : voff - vhalf;
    const uint8_t* vt = vh + (int64_t)kb0 * L::BPB;
    constexpr int nchunks = kD * L::CPR;
#pragma unroll
    for (int n = 0; n < (nchunks + kThreads - 1) / kThreads; ++n) {
      if ((kWaves * n + wave) * 64 < nchunks) {
        const uint8_t* src = vt + n * vstep + vo;
        uint8_t* dst = vsb + (kWaves * n + wave) * 64 * 16;
        if constexpr (L::CH == 16) lds_load16(src, dst);
        else lds_load12(src, dst);
      }
    }
  }
};

template <int VF, bool OUT_BF16, bool EFQ>
__global__ __launch_bounds__(kThreads, 2) void attention_fwd_mx(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs, int lq, int lk,
    float scale, int qtiles, void* __restrict__ o, float* __restrict__ row_max,
    float* __restrict__ row_sum, uint8_t* __restrict__ pc, uint8_t* __restrict__ ps) {
  using VL = VTile<VF>;
  // two buffers as separate LDS objects: the compiler can then tell that
  // loads streaming into one never alias reads of the other
  __shared__ __align__(16) uint8_t ks0[kKBytes], ks1[kKBytes];
  __shared__ __align__(16) uint8_t vsh0[kD * VL::CPR * 16], vsh1[kD * VL::CPR * 16];
  __shared__ uint8_t vsc0[kD * 2], vsc1[kD * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index through readfirstlane is known to be uniform, so the LDS
  // destinations of the direct loads (and all that depends only on the
  // wave) stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, h = lane >> 5;
  const int krow = kperm(col);  // this lane's A row of the score MFMAs

  // Workgroup order: the hardware deals consecutive workgroups round-robin
  // to the 8 XCDs, so renumber them to give each XCD a contiguous range of
  // (head, query tile) pairs; a head's K and V then stay in one L2.
  int wg = blockIdx.x;
  const int total = gridDim.x;
  if ((total & 7) == 0) wg = (wg & 7) * (total >> 3) + (wg >> 3);
  const int bh = wg / qtiles, qt = wg - bh * qtiles;
  const int qrow = qt * kRows + wave * 32 + col;
  const bool qvalid = qrow < lq;
  const int nbk = lk / 32;
  const int ntiles = (lk + kTile - 1) / kTile;

  // Q^T operand: lane holds d = 64h + 8i + e of its query, i = 0..7
  bf16x8_t qf[8];
  {
    const uint16_t* qp = q + ((int64_t)bh * lq + (qvalid ? qrow : 0)) * kD + 64 * h;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (qvalid) w = *reinterpret_cast<const u32x4_t*>(qp + 8 * i);
      qf[i] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x16_t acc[4];  // O^T tile T: d = 32T + 8(r/4) + 4h + r%4, query col
  f32x16_t lacc;    // every accumulator holds the query's l
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[0][r] = 0.0f; acc[1][r] = 0.0f; acc[2][r] = 0.0f; acc[3][r] = 0.0f;
    lacc[r] = 0.0f;
  }
  // running maxima: ms of the raw scores, m = fp32(ms * c) of t (scaling by
  // c > 0 keeps the order, so m is also the maximum of the fp32(S * c))
  const float c = scale * 0x1.715476p+0f;
  float ms = -INFINITY, m = -INFINITY;
  const i32x8_t ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};  // E2M1 1.0
  // the B operand of the PV products: E2M1 codes in dwords 0..3, the rest
  // unused by FP4 and kept zero across tiles
  i32x8_t pb = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t vlo, vhi;
  v_offsets<VF>(col, h, vlo, vhi);

  // V^T scale bytes of tile jt for row d = tid (tid < 128): the second
  // address repeats the first when the tile has one block, so both loads
  // are unconditional and nothing waits for them before they are stored
  const uint8_t* vs_head = vs + (int64_t)bh * kD * nbk;
  const uint32_t soff = (uint32_t)(tid * nbk);
  auto scale_ptr = [&](int jt) { return vs_head + 2 * jt + soff; };
  TileLoader<VF> loader;
  loader.init(k, vc, bh, lk, nbk, wave, lane);
  loader.issue(ks0, vsh0, 0);
  if (tid < kD) {
    const uint8_t* sp = scale_ptr(0);
    vsc0[2 * tid] = sp[0];
    vsc0[2 * tid + 1] = 1 < nbk ? sp[1] : (uint8_t)127;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // one 64-key tile: compute from (kt, vt, st) while tile j + 1 streams
  // into (kn, vn, sn)
  auto step = [&](int j, const uint8_t* kt, const uint8_t* vt, const uint8_t* st, uint8_t* kn,
                  uint8_t* vn, uint8_t* sn) __attribute__((always_inline)) {
    const int kb0 = 2 * j;
    const bool two = kb0 + 1 < nbk;  // false only for a last tile of 32 keys
    const bool two_next = kb0 + 3 < nbk;
    uint8_t sc_lo = 0, sc_hi = 0;
    if (j + 1 < ntiles) {
      loader.issue(kn, vn, j + 1);
      if (tid < kD) {
        const uint8_t* sp = scale_ptr(j + 1);
        sc_lo = sp[0];
        sc_hi = sp[two_next ? 1 : 0];
      }
    }

    // S^T of the tile: with the A rows in kperm order, s0[r] of lane half h
    // is key 32h + 8(r/4) + r%4 of the tile and s1[r] key 32h + 8(r/4) + 4 +
    // r%4
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // logical chunk 8h + i of rows kperm(col) and kperm(col) + 4, whose
      // kswz are both col % 16
      const int pch = ((8 * h + i) ^ (col & 15)) * 16;
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(kt + krow * 256 + pch);
      const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(kt + (krow + 4) * 256 + pch);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0), qf[i], s0, 0,
                                                   0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1), qf[i], s1, 0,
                                                   0, 0);
    }
    const bool dead = !two && h;  // the block past lk of a 32-key last tile

    // Tile maximum of the raw scores with NaN propagation (IEEE maximum): a
    // NaN score, or a running maximum whose t is infinite, sends the whole
    // wave through the careful path below; otherwise no shifted score can
    // be NaN.
    float mt = s0[0];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      mt = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mt, s0[r]), s1[r]);
    const float bmax = mt;  // the lane's block, NaN if any of its scores is
    mt = dead ? -INFINITY : mt;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const bool careful = __any(mt != mt || !(__builtin_fabsf(fmaxf(ms, mt) * c) < INFINITY));
    if (__builtin_expect(careful, 0)) {
      // the maximum the method defines skips NaN scores
      mt = s0[0];
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(fmaxf(mt, s0[r]), s1[r]);
      mt = dead ? -INFINITY : mt;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    ms = fmaxf(ms, mt);
    const float mnew = ms * c;
    const bool grow = mnew > m;
    if (__any(grow)) {
      const float alpha = grow ? exp2_ref_nonpos(m - mnew) : 1.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[0][r] *= alpha; acc[1][r] *= alpha; acc[2][r] *= alpha; acc[3][r] *= alpha;
      }
      lacc[0] *= alpha;  // the other 15 copies of l are never read
      m = grow ? mnew : m;
    }

    uint32_t byte;
    uint32_t pk[Fmt<F_E2M1>::W];
    if constexpr (!EFQ) {
      // every lane holds block h of the tile for its query: x[r] is key
      // 8(r/4) + r%4 of the block, y[r] is key 8(r/4) + 4 + r%4, in powers
      // of two
      float x[16], y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = s0[r] * c;
        y[r] = s1[r] * c;
      }
      // probabilities of the lane's 32-key block, in key order
      uint32_t v[32];
      if (careful) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * g + e] = __float_as_uint(exp2_ref_nonpos<true>(x[4 * g + e] - m));
            v[8 * g + 4 + e] = __float_as_uint(exp2_ref_nonpos<true>(y[4 * g + e] - m));
          }
      } else {
        // no NaN score and a finite maximum: the exp without its clamp,
        // checked below
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * g + e] = __float_as_uint(exp2_ref_nonpos_unclamped(x[4 * g + e] - m));
            v[8 * g + 4 + e] = __float_as_uint(exp2_ref_nonpos_unclamped(y[4 * g + e] - m));
          }
      }
      // p >= 0 or NaN, so the bit patterns order as the values and a NaN
      // orders above every finite one
      uint32_t amax = 0u;
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = max(amax, v[e]);
      if (__builtin_expect(!careful && __any(amax >= 0x7F800000u), 0)) {
        // a score of -inf (the only finite-maximum input the unclamped
        // sequence turns into NaN): the clamped exp2, for the whole wave
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * g + e] = __float_as_uint(exp2_ref_nonpos(x[4 * g + e] - m));
            v[8 * g + 4 + e] = __float_as_uint(exp2_ref_nonpos(y[4 * g + e] - m));
          }
        amax = 0u;
#pragma unroll
        for (int e = 0; e < 32; ++e) amax = max(amax, v[e]);
      }
      byte = scale_byte_from_amax<F_E2M1>(amax);
      // the four converts of a dword write its four bytes, so the dword's
      // previous contents do not matter: they start from pb's own dwords
      // (no register has to be cleared first)
      const float sc = scale_operand(byte);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w = (uint32_t)pb[q];
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(v[8 * q]),
                                                     __uint_as_float(v[8 * q + 1]), sc, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(v[8 * q + 2]),
                                                     __uint_as_float(v[8 * q + 3]), sc, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(v[8 * q + 4]),
                                                     __uint_as_float(v[8 * q + 5]), sc, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(v[8 * q + 6]),
                                                     __uint_as_float(v[8 * q + 7]), sc, 3);
        pk[q] = w;
      }
    } else {
      // EFQ reading, no exp, on u = t - m (already in powers of two): the
      // MX scale rule on 2^max u, and
      //   code = trunc(clamp(2 (u - (byte - 127)) + 2.5, 0, 7.5))
      // with the affine map taken from the raw score in one fused
      // multiply-add, a = fma(S, 2c, fp32((2.5 - 2 (byte - 127)) - 2m)).
      // max u = fp32(fp32(bmax c) - m) (both steps keep the order), NaN if
      // any u is (NaN score, or inf - inf), which poisons the block.
      const float U = bmax * c - m;
      // floor of max(U, -1000): every U below gives byte 0 as well
      const int E = (int)__builtin_floorf(__builtin_fmaxf(U, -1000.0f));
      const int b = min(max(E - Fmt<F_E2M1>::EMAX + 127, 0), 254);
      const float shift = (float)(b - 127);
      const float c2 = 2.0f * c;
      const float k2 = (2.5f - 2.0f * shift) - 2.0f * m;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = e < 4 ? s0[4 * j + e] : s1[4 * j + e - 4];
          const float cd = __builtin_amdgcn_fmed3f(__builtin_fmaf(sv, c2, k2), 0.0f, 7.5f);
          w |= (uint32_t)cd << (4 * e);
        }
        pk[j] = w;
      }
      byte = U != U ? 0xFFu : (uint32_t)b;
    }
    // blocks without codes: past lk (byte 0) and NaN blocks (0xFF), which
    // only a 32-key last tile or the careful path can produce (uniform)
    if (__builtin_expect(!two || careful, 0)) {
      const bool zero = dead || byte == 0xFFu;
      byte = dead ? 0u : byte;
#pragma unroll
      for (int e = 0; e < Fmt<F_E2M1>::W; ++e) pk[e] = zero ? 0u : pk[e];
    }
    pb[0] = (int)pk[0]; pb[1] = (int)pk[1]; pb[2] = (int)pk[2]; pb[3] = (int)pk[3];

#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int dd = 32 * T + col;
      const i32x8_t va = load_v_operand<VF>(vt, T, vlo, vhi);
      acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, acc[T], VF, 4, 0,
                                                               (int)st[2 * dd + h], 0, (int)byte);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, lacc, 4, 4, 0, 127, 0,
                                                           (int)byte);

    const int blk = 2 * j + h;
    if (pc != nullptr && qvalid && blk < nbk) {
      const int64_t b = ((int64_t)bh * lq + qrow) * nbk + blk;
      *reinterpret_cast<u32x4_t*>(pc + 16 * b) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
      ps[b] = (uint8_t)byte;
    }
    if (j + 1 < ntiles && tid < kD) {
      sn[2 * tid] = sc_lo;
      sn[2 * tid + 1] = two_next ? sc_hi : (uint8_t)127;
    }
    // the next tile has landed (own loads) and nobody reads this buffer
    // any more (barrier) before it is refilled
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(j, ks0, vsh0, vsc0, ks1, vsh1, vsc1);
    if (j + 1 < ntiles) step(j + 1, ks1, vsh1, vsc1, ks0, vsh0, vsc0);
  }

  if (!qvalid) return;
  const float l = lacc[0];
  const int64_t row = (int64_t)bh * lq + qrow;
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * T + 8 * g + 4 * h;
      float r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = acc[T][4 * g + e] / l;
        r4[e] = y != y ? __uint_as_float(0x7FC00000u) : y;
      }
      if constexpr (OUT_BF16) {
        u32x2_t w;
        w[0] = f32_to_bf16_rne(r4[0]) | (f32_to_bf16_rne(r4[1]) << 16);
        w[1] = f32_to_bf16_rne(r4[2]) | (f32_to_bf16_rne(r4[3]) << 16);
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o) + row * kD + d0) = w;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(o) + row * kD + d0) =
            make_float4(r4[0], r4[1], r4[2], r4[3]);
      }
    }
  if (h == 0) {
    if (row_max) row_max[row] = ms * scale;
    if (row_sum) row_sum[row] = l;
  }
}

template <int VF, bool EFQ>
hipError_t launch_vf(bool out_bf16, const void* q, const void* k, const void* vc,
                     const uint8_t* vs, int heads, int lq, int lk, float scale, void* o,
                     float* rm, float* rs, uint8_t* pc, uint8_t* ps, hipStream_t st) {
  const int qtiles = (lq + kRows - 1) / kRows;
  const dim3 grid((unsigned)(heads * qtiles)), block(kThreads);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint8_t* v8 = static_cast<const uint8_t*>(vc);
  if (out_bf16)
    hipLaunchKernelGGL((attention_fwd_mx<VF, true, EFQ>), grid, block, 0, st, q16, k16, v8, vs,
                       lq, lk, scale, qtiles, o, rm, rs, pc, ps);
  else
    hipLaunchKernelGGL((attention_fwd_mx<VF, false, EFQ>), grid, block, 0, st, q16, k16, v8, vs, lq,
                       lk, scale, qtiles, o, rm, rs, pc, ps);
  return hipGetLastError();
}

template <bool EFQ>
hipError_t launch_rule(int v_fmt, bool out_bf16, const void* q, const void* k,
                       const void* v_codes, const uint8_t* v_scales, int heads, int lq, int lk,
                       float scale, void* o, float* row_max, float* row_sum, uint8_t* pc,
                       uint8_t* ps, hipStream_t st) {
  switch (v_fmt) {
    case F_E4M3:
      return launch_vf<0, EFQ>(out_bf16, q, k, v_codes, v_scales, heads, lq, lk, scale, o,
                               row_max, row_sum, pc, ps, st);
    case F_E2M3:
      return launch_vf<2, EFQ>(out_bf16, q, k, v_codes, v_scales, heads, lq, lk, scale, o,
                               row_max, row_sum, pc, ps, st);
    case F_E3M2:
      return launch_vf<3, EFQ>(out_bf16, q, k, v_codes, v_scales, heads, lq, lk, scale, o,
                               row_max, row_sum, pc, ps, st);
    case F_E2M1:
      return launch_vf<4, EFQ>(out_bf16, q, k, v_codes, v_scales, heads, lq, lk, scale, o,
                               row_max, row_sum, pc, ps, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention(int v_fmt, bool efq, bool out_bf16, const void* q, const void* k,
                            const void* v_codes, const uint8_t* v_scales, int heads, int lq,
                            int lk, float scale, void* o, float* row_max, float* row_sum,
                            void* p_codes, uint8_t* p_scales, hipStream_t st) {
  uint8_t* pc = static_cast<uint8_t*>(p_codes);
  return efq ? launch_rule<true>(v_fmt, out_bf16, q, k, v_codes, v_scales, heads, lq, lk, scale,
                                 o, row_max, row_sum, pc, p_scales, st)
             : launch_rule<false>(v_fmt, out_bf16, q, k, v_codes, v_scales, heads, lq, lk, scale,
                                  o, row_max, row_sum, pc, p_scales, st);
}

}  // namespace mxk
