// HIP kernels for absorbed-MLA decode over fp8 (OCP E4M3 + one per-tensor
// scale) and bf16 KV caches on gfx950 (MI355X): the siblings of the MXFP4
// decode, on the same plan, partial format and reduce kernel.
//
// What is computed is the same definition as for the MXFP4 cache
// (kernelindex.com page "kernelbot-amd-mixed-mla-676098", _naive_fallback):
// softmax(sm_scale * q . K) V per sequence and head, V = the first 512 of the
// 576 dims. The caches are the ones of the same page: bf16 rows [T, 576]
// (_naive_fallback reads kv_data["bf16"]) and fp8 rows [T, 576] with one
// float32 scale for the whole tensor (_aiter_mla_decode: kv_fp8, kv_scale).
//
// Design (one workgroup of 4 waves per CU, one wave per SIMD, persistent over
// the planner's slots). These caches carry 2x (fp8) and 4x (bf16) the bytes
// per token of MXFP4, so each wave has ample issue time per byte and works
// alone, without the MXFP4 kernel's role split or workgroup barriers:
//  * A wave takes every 4th tile of its item (32 fp8 or 16 bf16 tokens, 18 KB
//    either way) into its own two LDS buffers with direct global->LDS
//    loads (18 x 1 KB, the rows copied as they sit in memory), issuing tile
//    i+1 before it waits for tile i; it waits only on its own loads.
//  * S^T = K Q^T with the 16 heads as the MFMA's N dimension:
//      - fp8: v_mfma_scale_f32_16x16x128_f8f6f4 on the e4m3 rows as stored
//        (A scale 1) against q split exactly into e4m3 hi + lo parts with one
//        power-of-two scale per (head, 128-dim chunk);
//      - bf16: v_mfma_f32_16x16x32_bf16 on the rows as stored.
//  * Online softmax in base 2 with the lazily raised running max of the
//    MXFP4 kernel (rescale only when a tile max exceeds it by more than 8),
//    P rounded to bf16, l summed from the rounded P.
//  * O += P V for all 512 dims (O in 128 registers) on the bf16 MFMA: V read
//    transposed from the same LDS rows (ds_read_b64_tr_b8 for fp8, then the
//    exact fp8 -> bf16 converter; ds_read_b64_tr_b16 for bf16, used as is).
//  * The 4 waves' (m, l, O) merge through LDS; a whole-sequence item writes
//    bf16 output, any other item a normalised fp32 partial and its base-2
//    LSE, which the MXFP4 library's reduce kernel merges.
//  * kGather: rows listed per token (kv_indices, page size 1); each wave
//    keeps the row indices of the next three tiles in an LDS ring.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
#define MLA_LDS __attribute__((address_space(3)))

constexpr int kHeads = MLA_NUM_HEADS;
constexpr int kQkDim = MLA_QK_DIM;
constexpr int kVDim = MLA_V_DIM;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = 18432;                 // one wave tile: 32 fp8 or 16 bf16 rows
constexpr int kDma = kTileBytes / 1024;           // 16-byte DMA instructions per tile (18)
constexpr int kOFrags = kVDim / 16;               // 32 output tiles of 16 dims
constexpr int kHalfFrag = kWaves * (kOFrags / 2) * 64 * 16;   // half the O tiles of all waves
constexpr int kLdsTotal = 2 * kWaves * kTileBytes;            // two tile buffers per wave (147456)
constexpr float kTau = 8.0f;
// Cache policy of the tile loads: non-temporal (nt); the rows are read once
// per call (12% faster than the default policy at B=256, kv=8192).
constexpr int kStream = 2;
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1.0e30f;

static_assert(kLdsTotal <= 160 * 1024, "LDS budget of one gfx950 CU");
static_assert(2 * kHalfFrag + 2 * kWaves * kHeads * 4 <= kLdsTotal, "the merge fits in the tile buffers");
static_assert(kTileBytes % 1024 == 0, "a tile is whole 1 KB DMA instructions");

template <bool kFp8>
struct Cfg {
  static constexpr int kRow = kFp8 ? kQkDim : 2 * kQkDim;   // bytes per token row
  static constexpr int kTile = kTileBytes / kRow;            // tokens per wave tile
  static constexpr int kSub = kTile / 16;                    // 16-token score blocks
  static constexpr int kStride = kWaves * kTile;             // a wave's step through the item
};
static_assert(Cfg<true>::kTile == 32 && Cfg<false>::kTile == 16, "tile shapes");

__device__ __forceinline__ f32x4_t mfma_bf16_k32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16_k16(const bf16x4_t& a, const bf16x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Stage the tile of `nvalid` valid rows starting at byte `src` into `buf`:
// 18 instructions, each writing 64 consecutive 16-byte LDS slots (lane i ->
// slot i, each lane choosing its global source). Slots past the last valid
// row repeat its last 16 bytes (finite data; those tokens get p = 0).
template <bool kFp8>
__device__ __forceinline__ void stage_tile(uint8_t* buf, const uint8_t* __restrict__ kv, int t0,
                                           int nvalid, int lane) {
  t0 = __builtin_amdgcn_readfirstlane(t0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const uint8_t* src = kv + (size_t)t0 * Cfg<kFp8>::kRow;
  const uint32_t lane_off = 16 * lane;
  if (nvalid >= Cfg<kFp8>::kTile) {
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + 1024 * i + lane_off),
                                       (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  } else {
    const uint32_t last = (uint32_t)(nvalid * Cfg<kFp8>::kRow - 16);
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + min(1024 * i + lane_off, last)),
                                       (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  }
}

// Wait until at most N of this wave's vector memory operations are in flight
// (they complete in order, so the older tile has landed).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS reads of the tile loop are issued from inline assembly, several per
// block, and waited for inside the same block: the compiler then sees no LDS
// read that could alias the direct loads in flight into the other buffer
// (it would otherwise wait for those loads too), and every output register
// holds its data when the block ends. Outputs are early-clobber so that no
// output shares the address register while reads are still being issued.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS uint8_t*)p;
}

// Nine 16-byte reads at addr + B + 64*j (j = 0..8).
template <int B>
__device__ __forceinline__ void lds_b128_x9(uint32_t addr, u32x4_t (&r)[9]) {
  asm volatile(
      "ds_read_b128 %0, %9 offset:%10\n\t"
      "ds_read_b128 %1, %9 offset:%11\n\t"
      "ds_read_b128 %2, %9 offset:%12\n\t"
      "ds_read_b128 %3, %9 offset:%13\n\t"
      "ds_read_b128 %4, %9 offset:%14\n\t"
      "ds_read_b128 %5, %9 offset:%15\n\t"
      "ds_read_b128 %6, %9 offset:%16\n\t"
      "ds_read_b128 %7, %9 offset:%17\n\t"
      "ds_read_b128 %8, %9 offset:%18\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7]), "=&v"(r[8])
      : "v"(addr), "i"(B), "i"(B + 64), "i"(B + 128), "i"(B + 192), "i"(B + 256), "i"(B + 320),
        "i"(B + 384), "i"(B + 448), "i"(B + 512));
}

// Eight transposing 8-bit (kTr16 false) or 16-bit (true) reads at
// addr + B + S*j (j = 0..7).
template <bool kTr16, int B, int S>
__device__ __forceinline__ void lds_tr_x8(uint32_t addr, i32x2_t (&v)[8]) {
  if constexpr (kTr16) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
          "=&v"(v[7])
        : "v"(addr), "i"(B), "i"(B + S), "i"(B + 2 * S), "i"(B + 3 * S), "i"(B + 4 * S), "i"(B + 5 * S),
          "i"(B + 6 * S), "i"(B + 7 * S));
  } else {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8 offset:%9\n\t"
        "ds_read_b64_tr_b8 %1, %8 offset:%10\n\t"
        "ds_read_b64_tr_b8 %2, %8 offset:%11\n\t"
        "ds_read_b64_tr_b8 %3, %8 offset:%12\n\t"
        "ds_read_b64_tr_b8 %4, %8 offset:%13\n\t"
        "ds_read_b64_tr_b8 %5, %8 offset:%14\n\t"
        "ds_read_b64_tr_b8 %6, %8 offset:%15\n\t"
        "ds_read_b64_tr_b8 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
          "=&v"(v[7])
        : "v"(addr), "i"(B), "i"(B + S), "i"(B + 2 * S), "i"(B + 3 * S), "i"(B + 4 * S), "i"(B + 5 * S),
          "i"(B + 6 * S), "i"(B + 7 * S));
  }
}

// ---- row lists and page tables (kv_indices) ------------------------------
// A wave keeps the row indices of four tiles in a ring of 128-byte slots
// after the tile buffers: the indices of tile i + 3 are loaded while tile
// i is computed, so those of tile i + 1 have landed when its rows are
// staged.
constexpr int kIdxSlot = 128;
constexpr int kIdxWave = 4 * kIdxSlot;
constexpr int kLdsGather = kLdsTotal + kWaves * kIdxWave;
static_assert(kLdsGather <= 160 * 1024, "LDS budget of one gfx950 CU");

// Row indices of a tile into `slot`, one 4-byte direct load per lane. The
// tile starts `rel0` tokens into its sequence, whose entries in `indices`
// start at `ibase`; tile row r (the last valid one repeated past the item's
// end) takes entry ibase + (rel0 + r) / ps, its page. A per-token row list
// is ps = 1 with ibase = the sequence's first token.
template <bool kFp8>
__device__ __forceinline__ void stage_idx(uint8_t* slot, const int32_t* __restrict__ indices, int ibase,
                                          int rel0, int nvalid, int ps, int lane) {
  ibase = __builtin_amdgcn_readfirstlane(ibase);
  rel0 = __builtin_amdgcn_readfirstlane(rel0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  if (lane < Cfg<kFp8>::kTile) {
    const int r = min(lane, nvalid - 1);
    const int e = ps == 1 ? ibase + rel0 + r : ibase + (int)((uint32_t)(rel0 + r) / (uint32_t)ps);
    __builtin_amdgcn_global_load_lds((const void*)(indices + e), (MLA_LDS void*)slot, 4, 0, 0);
  }
}

// Stage the tile whose row indices sit in `slot`: lane chunk c = 64*i + lane
// of instruction i is 16-byte chunk c % (row/16) of tile row c / (row/16)
// (rows past the item's end repeat the last valid row's last chunk). Lane r
// reads index r once (with pages, ps > 1, a page number that it turns into
// the pool row page * ps + the row's offset in its page); the DMA lanes take
// theirs by cross-lane permute, so the only LDS read is waited for inside
// its own block.
template <bool kFp8>
__device__ __forceinline__ void stage_gather(uint8_t* buf, const uint8_t* __restrict__ kv, const uint8_t* slot,
                                             int rel0, int nvalid, int ps, int lane) {
  using C = Cfg<kFp8>;
  constexpr int kCpr = C::kRow / 16;
  rel0 = __builtin_amdgcn_readfirstlane(rel0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const int last = min(nvalid, C::kTile) - 1;
  const int rl = min(lane, C::kTile - 1);
  uint32_t my;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(my)
               : "v"(lds_addr(slot) + 4u * (uint32_t)rl));
  if (ps != 1) my = my * (uint32_t)ps + (uint32_t)(rel0 + min(rl, last)) % (uint32_t)ps;
  uint32_t off[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int c = 64 * i + lane;
    int r = c / kCpr;
    int w = c - kCpr * r;
    if (r > last) {
      r = last;
      w = kCpr - 1;
    }
    const uint32_t phys = (uint32_t)__shfl((int)my, r);
    off[i] = phys * (uint32_t)C::kRow + 16u * (uint32_t)w;
  }
#pragma unroll
  for (int i = 0; i < kDma; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(kv + off[i]), (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
}

__device__ __forceinline__ float max_over_groups(float v) {
  // max over lanes h, h+16, h+32, h+48 (the 4 lane groups of head h); the
  // swap results are copied to scalars before their bit casts
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float m1 = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t u1 = __builtin_bit_cast(uint32_t, m1);
  const auto c = __builtin_amdgcn_permlane16_swap(u1, u1, false, false);
  const uint32_t c0 = c[0], c1 = c[1];
  return fmaxf(__builtin_bit_cast(float, c0), __builtin_bit_cast(float, c1));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// ---- Q operands --------------------------------------------------------

// fp8 cache: q of head `col` split exactly into e4m3 hi + lo on one E8M0
// pair per 128-dim chunk (sh puts the chunk's max |q| in [128, 256), sl =
// sh - 4). Lane group g holds, in the operand order of the 8-bit MFMA
// operands, dims 128m + 16g + (0..15) and 128m + 64 + 16g + (0..15) of chunk
// m (the same lane order as the K rows it meets, so the pairing is the
// identity whatever the matrix core's internal K order); chunk 4 is the 64
// rope dims 512 + 16g + (0..15) followed by zeros. The scale of a (head,
// chunk) is the same in all four lane groups, so it does not depend on how
// the matrix core maps scale lanes to K blocks.
struct QFp8 {
  i32x8_t hi[5], lo[5];
  uint32_t sh03, sl03, sh4, sl4;   // scale bytes: chunk m in byte m (chunks 0-3), chunk 4 in byte 0
};

__device__ __forceinline__ int e8m0_for_max(float mx) {
  const int ef = (int)(__builtin_bit_cast(uint32_t, mx) >> 23);
  return min(max(ef - 7, 0), 254);
}

// 16 floats on the E8M0 pair (sh, max(sh - 4, 0)) -> 4 dwords of hi codes
// and 4 of lo codes (hi + lo * 2^(sl - sh) = x * 2^(127 - sh) exactly for
// elements within 2^13 of the chunk max).
__device__ __forceinline__ void split16(const float* x, int sh, int32_t* hi, int32_t* lo) {
  const int sl = max(sh - 4, 0);
  const float inv = __builtin_bit_cast(float, (uint32_t)(254 - sh) << 23);
  const float up = __builtin_bit_cast(float, (uint32_t)(127 + sh - sl) << 23);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float h0 = x[4 * d] * inv, h1 = x[4 * d + 1] * inv;
    const float h2 = x[4 * d + 2] * inv, h3 = x[4 * d + 3] * inv;
    int hw = __builtin_amdgcn_cvt_pk_fp8_f32(h0, h1, 0, false);
    hw = __builtin_amdgcn_cvt_pk_fp8_f32(h2, h3, hw, true);
    const float r0 = __builtin_amdgcn_cvt_f32_fp8(hw, 0), r1 = __builtin_amdgcn_cvt_f32_fp8(hw, 1);
    const float r2 = __builtin_amdgcn_cvt_f32_fp8(hw, 2), r3 = __builtin_amdgcn_cvt_f32_fp8(hw, 3);
    int lw = __builtin_amdgcn_cvt_pk_fp8_f32((h0 - r0) * up, (h1 - r1) * up, 0, false);
    lw = __builtin_amdgcn_cvt_pk_fp8_f32((h2 - r2) * up, (h3 - r3) * up, lw, true);
    hi[d] = hw;
    lo[d] = lw;
  }
}

__device__ __forceinline__ void load16(const uint16_t* p, float* x) {
  const u32x4_t a = *(const u32x4_t*)p, b = *(const u32x4_t*)(p + 8);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_lo(a[k]);
    x[2 * k + 1] = bf16_hi(a[k]);
    x[8 + 2 * k] = bf16_lo(b[k]);
    x[8 + 2 * k + 1] = bf16_hi(b[k]);
  }
}

__device__ __forceinline__ QFp8 load_q_fp8(const uint16_t* qh, int grp) {
  QFp8 f;
  f.sh03 = f.sl03 = 0u;
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    float x[32];
    load16(qh + 128 * m + 16 * grp, x);
    if (m < 4) {
      load16(qh + 128 * m + 64 + 16 * grp, x + 16);
    } else {
#pragma unroll
      for (int k = 16; k < 32; ++k) x[k] = 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(x[k]));
    const int sh = e8m0_for_max(max_over_groups(mx));
    int32_t hi[8], lo[8];
    split16(x, sh, hi, lo);
    split16(x + 16, sh, hi + 4, lo + 4);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      f.hi[m][d] = hi[d];
      f.lo[m][d] = lo[d];
    }
    const uint32_t sl = (uint32_t)max(sh - 4, 0);
    if (m < 4) {
      f.sh03 |= (uint32_t)sh << (8 * m);
      f.sl03 |= sl << (8 * m);
    } else {
      f.sh4 = (uint32_t)sh;
      f.sl4 = sl;
    }
  }
  return f;
}

// bf16 cache: q of head `col` as the B operand of the bf16 16x16x32 MFMA,
// lane group g holding dims 32s + 8g + (0..7) of step s (18 steps).
struct QBf16 {
  bf16x8_t q[18];
};

__device__ __forceinline__ QBf16 load_q_bf16(const uint16_t* qh, int grp) {
  QBf16 f;
#pragma unroll
  for (int s = 0; s < 18; ++s) f.q[s] = *(const bf16x8_t*)(qh + 32 * s + 8 * grp);
  return f;
}

// ---- scores --------------------------------------------------------------

template <int M>
__device__ __forceinline__ f32x4_t mx8(const i32x8_t& k, const i32x8_t& q, uint32_t q_scales, f32x4_t acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, q, acc, 0, 0, 0, 127, M, (int32_t)q_scales);
}

// Raw scores (before the softmax scale) of tokens 16*sub + 4*grp + r for
// head `col`: S^T = K Q^T, A = 16 fp8 rows of the tile.
__device__ __forceinline__ f32x4_t scores_fp8(const uint8_t* buf, int sub, const QFp8& qo, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  u32x4_t r[9];   // chunk m: r[2m] = dims 128m + 16grp.., r[2m + 1] = 128m + 64 + 16grp..; r[8] = rope
  lds_b128_x9<0>(lds_addr(buf + (16 * sub + col) * Cfg<true>::kRow + 16 * grp), r);
  i32x8_t k[5];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    k[m] = i32x8_t{(int32_t)r[2 * m][0], (int32_t)r[2 * m][1], (int32_t)r[2 * m][2], (int32_t)r[2 * m][3],
                   (int32_t)r[2 * m + 1][0], (int32_t)r[2 * m + 1][1], (int32_t)r[2 * m + 1][2],
                   (int32_t)r[2 * m + 1][3]};
  k[4] = i32x8_t{(int32_t)r[8][0], (int32_t)r[8][1], (int32_t)r[8][2], (int32_t)r[8][3], 0, 0, 0, 0};
  f32x4_t h = {0.f, 0.f, 0.f, 0.f}, l = h;
  h = mx8<0>(k[0], qo.hi[0], qo.sh03, h);
  l = mx8<0>(k[0], qo.lo[0], qo.sl03, l);
  h = mx8<1>(k[1], qo.hi[1], qo.sh03, h);
  l = mx8<1>(k[1], qo.lo[1], qo.sl03, l);
  h = mx8<2>(k[2], qo.hi[2], qo.sh03, h);
  l = mx8<2>(k[2], qo.lo[2], qo.sl03, l);
  h = mx8<3>(k[3], qo.hi[3], qo.sh03, h);
  l = mx8<3>(k[3], qo.lo[3], qo.sl03, l);
  h = mx8<0>(k[4], qo.hi[4], qo.sh4, h);
  l = mx8<0>(k[4], qo.lo[4], qo.sl4, l);
  return h + l;
}

__device__ __forceinline__ f32x4_t scores_bf16(const uint8_t* buf, const QBf16& qo, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  const uint32_t a = lds_addr(buf + col * Cfg<false>::kRow + 16 * grp);
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  u32x4_t r[9];
  lds_b128_x9<0>(a, r);     // steps 0..8: dims 32s + 8grp..
#pragma unroll
  for (int s = 0; s < 9; ++s) {
    if (s & 1) a1 = mfma_bf16_k32(__builtin_bit_cast(bf16x8_t, r[s]), qo.q[s], a1);
    else a0 = mfma_bf16_k32(__builtin_bit_cast(bf16x8_t, r[s]), qo.q[s], a0);
  }
  lds_b128_x9<576>(a, r);   // steps 9..17
#pragma unroll
  for (int s = 0; s < 9; ++s) {
    if (s & 1) a0 = mfma_bf16_k32(__builtin_bit_cast(bf16x8_t, r[s]), qo.q[9 + s], a0);
    else a1 = mfma_bf16_k32(__builtin_bit_cast(bf16x8_t, r[s]), qo.q[9 + s], a1);
  }
  return a0 + a1;
}

// ---- P V -----------------------------------------------------------------

// fp8: O[16 heads][16 dims of block DB] += P[16][32 tokens] V[32][16]. Lane
// (col, grp) holds P of head col at its group's 8 tokens, K slot k <-> token
// 4*grp + (k & 3) + 16*(k >> 2); the transposing read gives it byte column
// (16*DB + col) of those 8 rows in the same order.
template <int G>
__device__ __forceinline__ void pv_fp8_group(uint32_t ta, const bf16x8_t& pa, f32x4_t (&o)[kOFrags]) {
  i32x2_t v[8];
  lds_tr_x8<false, 128 * G, 16>(ta, v);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[j][0], 1.0f, false);
    const bf16x2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[j][0], 1.0f, true);
    const bf16x2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[j][1], 1.0f, false);
    const bf16x2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[j][1], 1.0f, true);
    const bf16x8_t vb = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
    o[8 * G + j] = mfma_bf16_k32(pa, vb, o[8 * G + j]);
  }
}

__device__ __forceinline__ void pv_fp8(const uint8_t* buf, const bf16x8_t& pa, f32x4_t (&o)[kOFrags],
                                       int lane) {
  const int col = lane & 15, grp = lane >> 4;
  const int k = col >> 1;
  const int trow = 4 * grp + (k & 3) + 16 * (k >> 2);
  const uint32_t ta = lds_addr(buf + trow * Cfg<true>::kRow + 8 * (col & 1));
  pv_fp8_group<0>(ta, pa, o);
  pv_fp8_group<1>(ta, pa, o);
  pv_fp8_group<2>(ta, pa, o);
  pv_fp8_group<3>(ta, pa, o);
}

// bf16: O += P[16][16 tokens] V[16][16] per block; lane (col, grp) holds P
// of head col at tokens 4*grp + (0..3) and receives column (16*DB + col) of
// those 4 rows from the transposing 16-bit read.
template <int G>
__device__ __forceinline__ void pv_bf16_group(uint32_t ta, const bf16x4_t& pa, f32x4_t (&o)[kOFrags]) {
  i32x2_t v[8];
  lds_tr_x8<true, 256 * G, 32>(ta, v);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[8 * G + j] = mfma_bf16_k16(pa, __builtin_bit_cast(bf16x4_t, v[j]), o[8 * G + j]);
}

__device__ __forceinline__ void pv_bf16(const uint8_t* buf, const bf16x4_t& pa, f32x4_t (&o)[kOFrags],
                                        int lane) {
  const int col = lane & 15, grp = lane >> 4;
  const uint32_t ta = lds_addr(buf + (4 * grp + (col >> 2)) * Cfg<false>::kRow + 8 * (col & 3));
  pv_bf16_group<0>(ta, pa, o);
  pv_bf16_group<1>(ta, pa, o);
  pv_bf16_group<2>(ta, pa, o);
  pv_bf16_group<3>(ta, pa, o);
}

// One plan item: sequence, token range, partial index (-1: direct output).
struct __attribute__((aligned(16))) ItemWords {
  int32_t b, kb, ke, dest;
};
typedef const __attribute__((address_space(4))) int32_t ConstI32;

template <bool kFp8, bool kGather>
__global__ void __launch_bounds__(kThreads, 1)
mla_decode_dense_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                        const float* __restrict__ kv_scale, const int32_t* __restrict__ kv_indptr,
                        const int32_t* __restrict__ kv_indices, const int32_t* __restrict__ page_indptr,
                        int page_size, const int32_t* __restrict__ kv_start, uint16_t* __restrict__ out,
                        const int32_t* __restrict__ plan, float* __restrict__ part_lse,
                        float* __restrict__ part_out, float csc) {
  using C = Cfg<kFp8>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kGather ? kLdsGather : kLdsTotal];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // Header words in one batch (the compiler would fetch each only after the
  // previous check, a memory latency apiece).
  // Workgroups are dealt to the 8 XCDs in turn. When entries share rows
  // (kv_start), consecutive slots -- the query groups of one sequence --
  // go to workgroups of one XCD, so that its L2 serves the repeated reads.
  const bool xcd_order = !kGather && kv_start != nullptr && (gridDim.x & 7) == 0;
  const int first_slot = xcd_order ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                                   : (int)blockIdx.x;
  // The first slot's bounds (slot_indptr follows the header in both
  // planners' layouts, with an entry for every launched workgroup) and its
  // first item, from where it sits when the items follow slot_indptr of a
  // launch-sized plan with one item per slot before it, come in the same
  // batch; the item is used only if the header and slot_indptr confirm that
  // layout (the words read are inside the plan whatever it holds: it has at
  // least the launched number of slots, items from this offset on, and an
  // item per slot).
  const int32_t* slot_indptr = plan + MLA_PLAN_HEADER_WORDS;
  const int magic = plan[kPwMagic];
  const int version = plan[kPwVersion];
  const int num_slots = plan[kPwNumSlots];
  const int off_items = plan[kPwOffItems];
  const int i_begin0 = slot_indptr[first_slot];
  const int i_end0 = slot_indptr[first_slot + 1];
  const int spec_off = (MLA_PLAN_HEADER_WORDS + (int)gridDim.x + 1 + 3) & ~3;
  const ItemWords spec = *(const ItemWords*)(plan + spec_off + 4 * first_slot);
  asm volatile("" ::"s"(num_slots), "s"(off_items), "s"(i_begin0), "s"(i_end0), "s"(spec.b), "s"(spec.kb),
               "s"(spec.ke), "s"(spec.dest), "s"(q), "s"(kv), "s"(kv_indptr), "s"(out));
  // Only words written by a planner are followed: a workspace whose header
  // is not a plan of this version leaves the output untouched.
  if (magic != MLA_PLAN_MAGIC || version != MLA_PLAN_VERSION) return;
  // V scale and base-2 logit scale: the per-tensor fp8 scale multiplies both
  float vs = 1.0f;
  if constexpr (kFp8) vs = kv_scale[0];
  const float sc2 = csc * vs;

  const int32_t* items = plan + off_items;
  // kv_indptr is not written while the kernel runs: scalar loads through
  // the constant address space
  const ConstI32* kv_indptr_s = (const ConstI32*)kv_indptr;
  uint8_t* ring = lds + wave * (2 * kTileBytes);   // this wave's two tile buffers
  // merge area, over the tile buffers once every wave is done: the O tiles
  // of all waves, then the (m, l) statistics
  f32x4_t* frag = (f32x4_t*)lds;
  float* stats = (float*)(lds + 2 * kHalfFrag);

  for (int slot = first_slot; slot < num_slots; slot += gridDim.x) {
    const int i_begin = slot == first_slot ? i_begin0 : slot_indptr[slot];
    const int i_end = slot == first_slot ? i_end0 : slot_indptr[slot + 1];
    for (int it = i_begin; it < i_end; ++it) {
      const ItemWords iw = slot == first_slot && it == first_slot && off_items == spec_off
                               ? spec : *(const ItemWords*)(items + 4 * it);
      const int b = iw.b;
      const int dest = iw.dest;
      // bf16: q is requested before the bounds below are waited for (scalar
      // loads; the q loads are vector loads), so that it flies meanwhile
      const uint16_t* qh = q + ((size_t)b * kHeads + col) * kQkDim;
      QBf16 q16;
      if constexpr (!kFp8) q16 = load_q_bf16(qh, grp);
      // the item's rows, clamped to the sequence (a plan made for other
      // offsets reads nothing outside it)
      const int seq_lo = kv_indptr_s[b];
      const int kb = max(iw.kb, seq_lo);
      const int ke = min(iw.ke, kv_indptr_s[b + 1]);
      // first entry of the sequence in kv_indices: its page list, or its rows
      const int ibase = kGather && page_indptr != nullptr ? page_indptr[b] : seq_lo;
      // contiguous rows from kv_start[b] on, when given (shared by sequences)
      const uint8_t* kv_b = kv;
      if (!kGather && kv_start != nullptr) kv_b += ((ptrdiff_t)kv_start[b] - seq_lo) * C::kRow;
      // counts from differences, so that offsets near 2^31 - 1 cannot wrap;
      // a tile start is only formed for tiles inside the item (below ke)
      const int len = ke - kb;
      const int rel_first = C::kTile * wave;
      const int ntiles = rel_first < len ? (len - rel_first - 1) / C::kStride + 1 : 0;
      const int t_first = ntiles > 0 ? kb + rel_first : kb;

      // fp8: q is loaded and split chunk by chunk as it lands (measured
      // faster than splitting it whole under tile 0's flight)
      QFp8 q8;
      if constexpr (kFp8) q8 = load_q_fp8(qh, grp);
      float m = kMInit;    // running max of head col (base-2 scaled scores)
      float l = 0.f;       // this lane's share of head col's denominator
      f32x4_t o[kOFrags];
#pragma unroll
      for (int n = 0; n < kOFrags; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      __syncthreads();   // the previous item's merge has read the merge area
      // q has landed by now. Taking it here, before tile 0 is requested,
      // puts no wait for it in the loop (a wait for q after the tile's
      // loads would also wait for the tile).
      __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
      // Score tile i (landed in `buf`) and accumulate it into O.
      auto compute = [&](const uint8_t* buf, int i) {
        const int t0 = t_first + i * C::kStride;

        float x[4 * C::kSub];
        if constexpr (kFp8) {
#pragma unroll
          for (int s = 0; s < C::kSub; ++s) {
            const f32x4_t sv = scores_fp8(buf, s, q8, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) x[4 * s + r] = sv[r];
          }
        } else {
          const f32x4_t sv = scores_bf16(buf, q16, lane);
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = sv[r];
        }
#pragma unroll
        for (int j = 0; j < 4 * C::kSub; ++j) x[j] *= sc2;
        const int nvalid = ke - t0;   // a difference: no wrap near 2^31 - 1
        if (nvalid < C::kTile) {   // tail tile: tokens past the item get p = 0
#pragma unroll
          for (int s = 0; s < C::kSub; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * s + 4 * grp + r >= nvalid) x[4 * s + r] = kNegInf;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 4 * C::kSub; ++j) mx = fmaxf(mx, x[j]);
        mx = max_over_groups(mx);
        const bool need = mx > m + kTau;
        if (__ballot(need)) {
          const float m_new = need ? mx : m;
          const float alpha = need ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
          m = m_new;
          l *= alpha;
          f32x4_t ar;
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * grp + r);
#pragma unroll
          for (int n = 0; n < kOFrags; ++n) o[n] *= ar;
        }
        float p[4 * C::kSub];
#pragma unroll
        for (int j = 0; j < 4 * C::kSub; ++j) {
          p[j] = (float)(__bf16)__builtin_amdgcn_exp2f(x[j] - m);
          l += p[j];
        }
        if constexpr (kFp8) {
          const bf16x8_t pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                               (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
          pv_fp8(buf, pa, o, lane);
        } else {
          const bf16x4_t pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
          pv_bf16(buf, pa, o, lane);
        }
      };
      if constexpr (kGather) {
        // Per iteration the wave issues the rows of tile i + 1 (18 loads)
        // and the indices of tile i + 3 (1 load; past the item's last tile
        // they repeat its indices, so the counts below never change).
        uint8_t* islot = lds + kLdsTotal + wave * kIdxWave;
        auto tile_t0 = [&](int k) { return t_first + min(k, ntiles - 1) * C::kStride; };
        if (ntiles > 0) {
          stage_idx<kFp8>(islot, kv_indices, ibase, tile_t0(0) - seq_lo, ke - tile_t0(0), page_size, lane);
          stage_idx<kFp8>(islot + kIdxSlot, kv_indices, ibase, tile_t0(1) - seq_lo, ke - tile_t0(1), page_size,
                          lane);
          wait_vm<0>();
          stage_gather<kFp8>(ring, kv, islot, t_first - seq_lo, ke - t_first, page_size, lane);
          stage_idx<kFp8>(islot + 2 * kIdxSlot, kv_indices, ibase, tile_t0(2) - seq_lo, ke - tile_t0(2),
                          page_size, lane);
        }
        for (int i = 0; i < ntiles; ++i) {
          if (i + 1 < ntiles) {
            wait_vm<kDma + 1>();   // indices of tile i + 1 (then: rows of i, indices of i + 2)
            const int tn = t_first + (i + 1) * C::kStride;
            stage_gather<kFp8>(ring + ((i + 1) & 1) * kTileBytes, kv, islot + ((i + 1) & 3) * kIdxSlot,
                               tn - seq_lo, ke - tn, page_size, lane);
            stage_idx<kFp8>(islot + ((i + 3) & 3) * kIdxSlot, kv_indices, ibase, tile_t0(i + 3) - seq_lo,
                            ke - tile_t0(i + 3), page_size, lane);
            wait_vm<kDma + 2>();   // rows of tile i (then: indices of i + 2, rows of i + 1, indices of i + 3)
          } else {
            wait_vm<0>();
          }
          compute(ring + (i & 1) * kTileBytes, i);
        }
      } else {
        if (ntiles > 0) stage_tile<kFp8>(ring, kv_b, t_first, ke - t_first, lane);
        for (int i = 0; i < ntiles; ++i) {
          // tile i + 1 goes into the other buffer before tile i is waited for
          if (i + 1 < ntiles) {
            const int tn = t_first + (i + 1) * C::kStride;
            stage_tile<kFp8>(ring + ((i + 1) & 1) * kTileBytes, kv_b, tn, ke - tn, lane);
            wait_vm<kDma>();
          } else {
            wait_vm<0>();
          }
          compute(ring + (i & 1) * kTileBytes, i);
        }
      }

      // ---- merge the 4 waves' states ----
      float lh = l + __shfl_xor(l, 16);
      lh += __shfl_xor(lh, 32);
      __syncthreads();   // every wave is done with its tile buffers
      if (grp == 0) {
        stats[(2 * wave) * kHeads + col] = m;
        stats[(2 * wave + 1) * kHeads + col] = lh;
      }
#pragma unroll
      for (int f = 0; f < kOFrags; ++f) frag[(wave * kOFrags + f) * 64 + lane] = o[f];
      __syncthreads();

      float wgt[4][kWaves], inv[4], lse[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        float mw[kWaves], lw[kWaves];
        float mmax = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          mw[w] = stats[(2 * w) * kHeads + h];
          lw[w] = stats[(2 * w + 1) * kHeads + h];
          if (lw[w] != 0.f) mmax = fmaxf(mmax, mw[w]);
        }
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          wgt[r][w] = lw[w] != 0.f ? __builtin_amdgcn_exp2f(mw[w] - mmax) : 0.f;
          lsum += wgt[r][w] * lw[w];
        }
        inv[r] = lsum != 0.f ? vs / lsum : 0.f;
        lse[r] = lsum != 0.f ? mmax + __builtin_amdgcn_logf(lsum) : kNegInf;
      }
      // wave w writes output tiles 8w .. 8w + 7 (dims 128w .. 128w + 127)
#pragma unroll
      for (int f = 0; f < kOFrags / kWaves; ++f) {
        const int blk = (kOFrags / kWaves) * wave + f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const f32x4_t fr = frag[(w * kOFrags + blk) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] += wgt[r][w] * fr[r];
        }
        const int d = 16 * blk + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 4 * grp + r;
          const float v = acc[r] * inv[r];
          if (dest < 0) {
            out[((size_t)b * kHeads + h) * kVDim + d] = __builtin_bit_cast(uint16_t, (__bf16)v);
          } else {
            part_out[((size_t)dest * kHeads + h) * kVDim + d] = v;
          }
        }
      }
      if (dest >= 0 && wave == 0 && col == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) part_lse[(size_t)dest * kHeads + 4 * grp + r] = lse[r];
      }
    }
  }
}

}  // namespace

size_t decode_dense_lds_bytes() { return (size_t)kLdsGather; }

template <bool kFp8, bool kGather>
static void launch_dense(const DecodeArgs& a, const float* kv_scale, void* stream) {
  hipLaunchKernelGGL((mla_decode_dense_kernel<kFp8, kGather>), dim3(a.grid), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint16_t*)a.q, a.kv_packed, kv_scale, a.kv_indptr, a.kv_indices,
                     kGather ? a.page_indptr : (const int32_t*)nullptr, kGather ? a.page_size : 1,
                     kGather ? (const int32_t*)nullptr : a.kv_start, (uint16_t*)a.out, a.plan, a.part_lse,
                     a.part_out, a.score_scale_log2);
}

int launch_decode_dense(const DecodeArgs& a, bool fp8, const float* kv_scale, void* stream) {
  if (a.num_slots <= 0 || a.grid <= 0) return (int)hipSuccess;
  const bool gather = a.kv_indices != nullptr;
  if (fp8) {
    if (gather) launch_dense<true, true>(a, kv_scale, stream);
    else launch_dense<true, false>(a, kv_scale, stream);
  } else {
    if (gather) launch_dense<false, true>(a, kv_scale, stream);
    else launch_dense<false, false>(a, kv_scale, stream);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
