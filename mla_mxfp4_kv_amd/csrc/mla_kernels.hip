// HIP kernels for MXFP4-KV absorbed-MLA decode on gfx950 (MI355X).
//
// What is computed (kernelindex.com "amd-mixed-mla" pages): for one query
// token per sequence and 16 heads, softmax(sm_scale * q . K) V over the
// sequence's tokens, where K is the 576-wide MXFP4-decoded latent+rope row
// and V its first 512 dims ("kernelbot-amd-mixed-mla-676098",
// _naive_fallback). The split-K structure -- partial (acc, LSE) per KV range,
// then an LSE-weighted merge -- is the one of the 608791 page (stage-1 and
// reduce kernels) and of the 676098 page (partial and reduce kernels).
//
// Design for CDNA4 (8 waves per workgroup = 2 per SIMD, one workgroup per
// CU, persistent over the planner's slots):
//  * The workgroup's KV range is cut into 32-token tiles interleaved over 4
//    wave pairs; the two waves of a pair share a SIMD and each tile, and
//    split its work by role. Packed rows (288 B, as in memory) and the
//    E8M0 rows (18 B, as the 16-byte chunks that cover them) go straight
//    from HBM into the pair's LDS ring of three tile buffers with direct
//    global->LDS loads, one tile ahead of the one being scored.
//  * One workgroup barrier per round: in round i the scorer wave computes
//    S for tile i while the P V wave accumulates tile i-1, so the matrix
//    core of the SIMD takes one wave's products while the other decodes or
//    exponentiates.
//  * Scorer: S^T = K Q^T with the 16 heads as the MFMA's N dimension. The
//    512 latent dims run on v_mfma_scale_f32_16x16x128_f8f6f4 with the
//    packed fp4 rows and their E8M0 bytes as the scaled A operand and q as
//    an exact hi + lo pair of e4m3 operands with per-block scales; the 64
//    rope dims on v_mfma_f32_16x16x32_bf16 after v_cvt_scalef32_pk_bf16_fp4
//    (exactly e2m1 * 2^(e-127)). Then the online softmax in base 2 with a
//    lazily updated running max (rescale only when a tile max exceeds it by
//    more than 8), and the V scales rewritten as converter operands.
//  * P V wave: O += P V for all 512 latent dims (O in 128 registers) on the
//    bf16 MFMA. V comes from the packed LDS tile through ds_read_b64_tr_b8
//    (8 tokens x 1 byte per lane) and is decoded with each token's scale
//    into (even dim, odd dim) pairs; v_perm_b32 regroups them into token
//    pairs, so the even and odd latent dims of a 32-dim scale block are two
//    output tiles with the whole tile's 32 tokens as K.
//  * The 4 pairs' (m, l, O) are merged through LDS; a whole-sequence item
//    writes bf16 output directly, any other item writes a normalised fp32
//    partial and its base-2 LSE for the reduce kernel.
//  * kGather: the same kernel over a cache whose rows are listed per token
//    (kv_indices, page size 1, as the 676098 page passes its decode): the
//    scorer stages each tile's row indices a round ahead and the tile's rows
//    and per-row scale chunks are gathered through them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
#define MLA_LDS __attribute__((address_space(3)))

constexpr int kHeads = MLA_NUM_HEADS;
constexpr int kQkDim = MLA_QK_DIM;
constexpr int kVDim = MLA_V_DIM;
constexpr int kRowBytes = MLA_PACKED_BYTES;     // 288
constexpr int kBlocks = MLA_SCALES_PER_TOKEN;   // 18
constexpr int kWaves = 8;                       // 4 pairs x 2 halves, 2 waves per SIMD
constexpr int kPairs = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                       // tokens per pair step
constexpr int kTileStride = kPairs * kTile;     // a pair's step through the range
constexpr int kNumBuf = 3;                      // LDS tile buffers per pair: P V, QK, in flight
constexpr int kLdsRow = kRowBytes;              // packed rows as in memory: a tile is one contiguous copy
constexpr int kRowDma = kTile * kRowBytes / 1024;  // 16-byte DMA instructions per tile (9)
constexpr int kLdsRaw = kTile * kRowBytes;      // raw E8M0 rows of the tile after the packed rows
constexpr int kRawChunks = (kTile * kBlocks + 15) / 16 + 1;  // 16-byte chunks covering them at any alignment (37)
constexpr int kLdsBuf = kLdsRaw + kRawChunks * 16 + 48;      // 9856 (multiple of 64)
constexpr int kLdsPair = kNumBuf * kLdsBuf;
constexpr int kVBlocks = kVDim / 32;            // 16 scale blocks of V
constexpr int kFmtTile = kVBlocks * kTile * 4;  // one tile's V scales as exponent-field dwords
constexpr int kLdsFmt = kPairs * kLdsPair;      // [parity][pair][block][position] dwords
constexpr int kLdsXchg = kLdsFmt + 2 * kPairs * kFmtTile;   // tile hand-offs: [parity][pair][lane]
constexpr int kLdsMain = kLdsXchg + 2 * kPairs * 64 * 32;
constexpr int kMergeFrag = kPairs * 32 * 64 * 16;   // O fragments: [pair][fragment][lane]
constexpr int kMergeBytes = kMergeFrag + kPairs * 2 * kHeads * 4;
constexpr int kLdsTotal = (kLdsMain > kMergeBytes) ? kLdsMain : kMergeBytes;
constexpr float kTau = 8.0f;                    // lazy-rescale threshold (base-2 units)
// Cache policy of the tile loads: non-temporal (nt). The cache is read once
// per call, and marking the stream non-temporal measured 6% faster for this
// kernel and 12% for the fp8/bf16 ones at B=256, kv=8192 (same process,
// interleaved) than the default policy; the scope bits (sc0/sc1) changed
// nothing.
constexpr int kStream = 2;
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1.0e30f;              // running max before the first tile (finite: no inf - inf)

static_assert(kLdsTotal <= 160 * 1024, "LDS budget of one gfx950 CU");
static_assert(kTile * kRowBytes % 1024 == 0, "a tile's rows are whole 1 KB DMA instructions");

// LDS layout by cache addressing. kGather (rows listed per token in
// kv_indices) keeps each tile row's scale bytes in a 32-byte slot of its own
// (the two aligned 16-byte chunks that cover them) and the tile's 32 row
// indices after them; the contiguous layout is the one above.
template <bool kGather>
struct Lds {
  static constexpr int kBuf = kGather ? kLdsRaw + kTile * 32 + kTile * 4 : kLdsBuf;
  static constexpr int kIdx = kLdsRaw + kTile * 32;
  static constexpr int kPair = kNumBuf * kBuf;
  static constexpr int kFmt = kPairs * kPair;
  static constexpr int kXchg = kFmt + 2 * kPairs * kFmtTile;
  static constexpr int kMain = kXchg + 2 * kPairs * 64 * 32;
  static constexpr int kTotal = kMain > kMergeBytes ? kMain : kMergeBytes;
};
static_assert(Lds<false>::kTotal == kLdsTotal, "contiguous layout unchanged");
static_assert(Lds<true>::kTotal <= 160 * 1024, "LDS budget of one gfx950 CU");
static_assert(Lds<true>::kBuf % 64 == 0, "buffers stay 64-byte aligned");

// Stage one 32-token tile into an LDS buffer with direct global->LDS loads
// (a 16-byte DMA instruction writes 64 consecutive 16-byte LDS slots, lane i
// -> slot i, each lane choosing its global source):
//  * rows: the tile's 32 packed rows are one contiguous 9 KB range, copied
//    as is (row stride 288 bytes) by nine instructions; in a tile that ends
//    the item, slots past its last valid row repeat that row's last 16
//    bytes (finite fp4 codes; those tokens get p = 0);
//  * scales: the tile's 18-byte E8M0 rows are contiguous too; the 16-byte-
//    aligned chunks that cover them are copied (37 lanes), so byte (row,
//    blk) lands at raw + delta + 18*row + blk with delta = the start's
//    offset in its chunk. Chunks past the last valid byte repeat the last
//    one; aligned chunks of valid bytes never cross a page.
// Only the pair's scorer issues them (issued by all waves at once, the
// instructions queue in the CU's address unit and stall every issuer).

// Offset of a tile's first scale byte inside its 16-byte chunk.
__device__ __forceinline__ int raw_delta(const uint8_t* sc, int t0) {
  return (int)((uintptr_t)(sc + (size_t)t0 * kBlocks) & 15);
}

// Issue DMA instructions kFirst .. kFirst + kCount - 1 of the tile starting
// at token t0 (`nvalid` = tokens of the tile inside the item), and with
// kScales the one for its scale rows.
template <int kFirst, int kCount, bool kScales>
__device__ __forceinline__ void stage_dma(uint8_t* buf, const uint8_t* __restrict__ kv,
                                          const uint8_t* __restrict__ sc, int t0, int nvalid,
                                          int lane) {
  // t0 and nvalid are wave-uniform: the tile base goes in SGPRs and each lane
  // only adds its 32-bit slot offset.
  t0 = __builtin_amdgcn_readfirstlane(t0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const uint8_t* kv_t = kv + (size_t)t0 * kRowBytes;
  const uint32_t lane_off = 16 * lane;
  if (nvalid >= kTile) {
#pragma unroll
    for (int i = kFirst; i < kFirst + kCount; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(kv_t + 1024 * i + lane_off),
                                       (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  } else {
    const uint32_t last = (uint32_t)(nvalid * kRowBytes - 16);
#pragma unroll
    for (int i = kFirst; i < kFirst + kCount; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(kv_t + min(1024 * i + lane_off, last)),
                                       (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  }
  if constexpr (kScales) {
    const uintptr_t first = (uintptr_t)(sc + (size_t)t0 * kBlocks);
    const uintptr_t last_chunk = (first + (uintptr_t)(kBlocks * min(nvalid, kTile)) - 1) & ~(uintptr_t)15;
    const uintptr_t src = min((first & ~(uintptr_t)15) + lane_off, last_chunk);
    if (lane < kRawChunks)
      __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(buf + kLdsRaw), 16, 0, kStream);
  }
}

// The whole tile.
__device__ __forceinline__ void stage_dma(uint8_t* buf, const uint8_t* __restrict__ kv,
                                          const uint8_t* __restrict__ sc, int t0, int nvalid,
                                          int lane) {
  stage_dma<0, kRowDma, true>(buf, kv, sc, t0, nvalid, lane);
}

// Row indices of the tile starting at token t0 (kv_indices[t0 .. t0 + 31],
// the last valid one repeated past the item's end) into the buffer's index
// slot: one 4-byte direct load per lane of the first 32.
__device__ __forceinline__ void stage_idx(uint8_t* buf, const int32_t* __restrict__ kv_indices, int t0,
                                          int nvalid, int lane) {
  t0 = __builtin_amdgcn_readfirstlane(t0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  if (lane < kTile) {
    const int r = min(lane, nvalid - 1);
    __builtin_amdgcn_global_load_lds((const void*)(kv_indices + t0 + r),
                                     (MLA_LDS void*)(buf + Lds<true>::kIdx), 4, 0, 0);
  }
}

// Page tables: the row of tile row r (lanes 0..31; the last valid row
// repeated past the item's end) is page * ps + x % ps with x = rel0 + r its
// token's position in the sequence and page = indices[ibase + x / ps]. The
// page entries are loaded into registers a round before the rows are
// needed, and stored as rows into the index slot just before the tile is
// staged, so every later reader of the slot sees rows.
struct PageRows {
  uint32_t page;   // the token's page (in flight until the next round)
  uint32_t off;    // its row within the page
};

__device__ __forceinline__ PageRows load_pages(const int32_t* __restrict__ indices, int ibase, int rel0,
                                               int nvalid, int ps, int lane) {
  rel0 = __builtin_amdgcn_readfirstlane(rel0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const uint32_t x = (uint32_t)(rel0 + min(min(lane, kTile - 1), nvalid - 1));
  const uint32_t pg = x / (uint32_t)ps;
  PageRows r;
  r.off = x - pg * (uint32_t)ps;
  r.page = (uint32_t)indices[ibase + (int)pg];
  return r;
}

__device__ __forceinline__ void store_page_rows(uint8_t* buf, const PageRows& r, int ps, int lane) {
  if (lane < kTile) ((int32_t*)(buf + Lds<true>::kIdx))[lane] = (int32_t)(r.page * (uint32_t)ps + r.off);
}

// Stage a tile whose rows are listed in the buffer's index slot: lane chunk
// c = 64*i + lane of instruction i is 16-byte chunk c % 18 of tile row c / 18
// (rows past the item's end repeat the last valid row's last chunk); each
// row's 18 scale bytes come as the two aligned 16-byte chunks that cover
// them (an 18-byte row starts at an even offset, so two always suffice)
// into the row's 32-byte slot. All indices are read before any load is
// issued.
__device__ __forceinline__ void stage_gather(uint8_t* buf, const uint8_t* __restrict__ kv,
                                             const uint8_t* __restrict__ sc, int nvalid, int lane) {
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const int last = min(nvalid, kTile) - 1;
  const int32_t* idx = (const int32_t*)(buf + Lds<true>::kIdx);
  uint32_t off[kRowDma];
#pragma unroll
  for (int i = 0; i < kRowDma; ++i) {
    const int c = 64 * i + lane;
    int r = c / 18;
    int w = c - 18 * r;
    if (r > last) {
      r = last;
      w = 17;
    }
    off[i] = (uint32_t)idx[r] * (uint32_t)kRowBytes + 16u * (uint32_t)w;
  }
  const uintptr_t srow = (uintptr_t)(sc + (size_t)(uint32_t)idx[min(lane >> 1, last)] * kBlocks);
#pragma unroll
  for (int i = 0; i < kRowDma; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(kv + off[i]), (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  __builtin_amdgcn_global_load_lds((const void*)((srow & ~(uintptr_t)15) + 16 * (uintptr_t)(lane & 1)),
                                   (MLA_LDS void*)(buf + kLdsRaw), 16, 0, kStream);
}

// LDS address of the scale bytes of tile row `row`. delta: in the
// contiguous layout the offset of the tile's first scale byte in its
// 16-byte chunk; with kGather the offset of the scale array's base in its
// chunk (row p starts 18 p = 2 p mod 16 bytes after it).
template <bool kGather>
__device__ __forceinline__ const uint8_t* scale_row(const uint8_t* buf, int delta, int row) {
  if constexpr (kGather) {
    const int32_t* idx = (const int32_t*)(buf + Lds<true>::kIdx);
    return buf + kLdsRaw + 32 * row + ((delta + 2 * idx[row]) & 15);
  } else {
    return buf + kLdsRaw + delta + kBlocks * row;
  }
}

// Rewrite the V scales of a landed tile as exponent-field dwords (e << 23,
// the form the fp4 converter takes as its scale operand) into `fmt`
// ([block][position]). Position 8g + j of a block is token 4g + j of the
// first 16-token sub-tile for j < 4 and token 16 + 4g + j - 4 of the second
// for j >= 4: the order in which lane group g holds its 8 probabilities.
// `l` (0..127) picks one block and four consecutive positions. Rows at or
// past `nvalid` get scale 1 (their p is 0, and a stale byte must not turn
// 0 * V into NaN).
template <bool kGather>
__device__ __forceinline__ void format_scales(const uint8_t* buf, uint8_t* fmt, int delta,
                                              int nvalid, int l) {
  const int blk = l >> 3;
  const int pg = l & 7;
  const int row0 = 16 * (pg & 1) + 4 * (pg >> 1);
  u32x4_t v;
  if constexpr (kGather) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = scale_row<true>(buf, delta, row0 + j)[blk];
      v[j] = row0 + j < nvalid ? e << 23 : 127u << 23;
    }
  } else {
    const uint8_t* raw = buf + kLdsRaw + delta + blk;
    if (nvalid >= kTile) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (uint32_t)raw[kBlocks * (row0 + j)] << 23;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t e = raw[kBlocks * (row0 + j)];
        v[j] = row0 + j < nvalid ? e << 23 : 127u << 23;
      }
    }
  }
  *(u32x4_t*)(fmt + blk * (kTile * 4) + 16 * pg) = v;
}

// LDS reads issued from inline assembly: the compiler does not count them,
// so their results are only used after an explicit lgkmcnt wait that names
// the destination registers.
template <int kOff>
__device__ __forceinline__ u32x2_t lds_tr8(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff));
  return r;
}
template <int kOff>
__device__ __forceinline__ u32x4_t lds_b128(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff));
  return r;
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS uint8_t*)p;
}

// Wait for this wave's share of the DMA in flight (vector memory operations
// complete in order). The memory clobber keeps later LDS reads below it.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 8 e2m1 codes (one dword, low nibble first) times 2^(e-127) -> 8 bf16.
// The converter reads only the exponent field of the scale operand.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ float exp_field(uint32_t e8m0) {
  return __builtin_bit_cast(float, e8m0 << 23);
}

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Running softmax statistics of the 16 heads, held by the wave that
// computes the scores.
struct SoftmaxState {
  f32x4_t l;         // denominator of heads 4*grp + r (C layout, any column)
  float m;           // running max (base-2 scaled scores) of head `col`
};

// What the score wave hands the P V wave for one tile: P in the A-operand
// layout of the bf16 MFMA (lane: head `col`, tokens of lane group `grp` in
// the order of the formatted scales) and the factor that rescales O's rows
// (heads 4*grp + r) before this tile is added (1 when the max is kept).
struct TileHandoff {
  u32x4_t p;
  f32x4_t alpha;
};

// max(a, b, c) in one instruction (maxNum semantics, as fmaxf).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max over the 4 lanes that hold the same head (lanes h, h+16, h+32, h+48).
__device__ __forceinline__ float max_over_groups(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  // The swap results are copied to scalars before the bit casts: a bit cast
  // of an element of the builtin's two-element result reads element 0 for
  // both, which silently turned this reduction into a copy of lane group 0.
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float m1 = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t u1 = __builtin_bit_cast(uint32_t, m1);
  const auto c = __builtin_amdgcn_permlane16_swap(u1, u1, false, false);
  const uint32_t c0 = c[0], c1 = c[1];
  return fmaxf(__builtin_bit_cast(float, c0), __builtin_bit_cast(float, c1));
}

// Q of one sequence in the operand forms of S^T = K Q^T (lane: head `col`,
// lane group `grp`).
//  * Latent dims 0..511 feed v_mfma_scale_f32_16x16x128_f8f6f4 with the fp4
//    K rows as A: lane group g of A holds the 32 consecutive dims
//    128m + 32g.. of chunk m (one E8M0 block, whose byte is g's A scale).
//    The matrix core pairs those nibbles with B bytes such that B lane group
//    g' must hold dims 128m + 16g' + (0..15) and 128m + 64 + 16g' + (0..15),
//    and B's scale from lane group g' applies to the B values paired with A
//    group g' -- Q block 128m + 32g'.. . So a lane converts its two 16-value
//    halves with the scales of blocks g'/2 and 2 + g'/2 and supplies block
//    g''s scale byte.
//  * Each bf16 q is split exactly into hi * 2^(sh-127) + lo * 2^(sl-127),
//    hi and lo e4m3 (a bf16 mantissa has 8 bits, an e4m3 one 4): sh puts the
//    block max in [128, 256), sl = sh - 4 (clamped at 0). Byte m of sc_hi /
//    sc_lo holds the supplied sh / sl of chunk m.
//  * Rope dims 512..575 stay bf16 for v_mfma_f32_16x16x32_bf16.
struct QOperands {
  i32x8_t hi[4];
  i32x8_t lo[4];
  uint32_t sc_hi, sc_lo;
  bf16x8_t rope[2];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ int e8m0_for_max(float mx) {
  const int ef = (int)(__builtin_bit_cast(uint32_t, mx) >> 23);  // biased exponent of the max
  return min(max(ef - 7, 0), 254);
}

// 16 floats -> 16 e4m3 hi bytes and 16 e4m3 lo bytes (4 dwords each) on the
// E8M0 pair (sh, sh - 4 clamped).
__device__ __forceinline__ void split16(const float* x, int sh, int* hi, int* lo) {
  const int sl = max(sh - 4, 0);
  const float inv = __builtin_bit_cast(float, (uint32_t)(254 - sh) << 23);      // 2^(127 - sh)
  const float up = __builtin_bit_cast(float, (uint32_t)(127 + sh - sl) << 23);  // 2^(sh - sl)
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

// The q operands are built once per item by the four scorer waves together:
// wave `pair` loads and splits the 128-dim chunk m = pair for all 16 heads
// and leaves it in LDS, then every scorer reads all four chunks back. The
// lane's pieces of chunk m as loaded: 4 x 16 bytes (and the 64 rope dims,
// which every scorer loads for itself).
struct QChunk {
  u32x4_t w[4];
  u32x4_t rope[2];
};

__device__ __forceinline__ QChunk load_q_chunk(const uint16_t* qh, int m, int grp) {
  QChunk c;
  const u32x4_t* p0 = (const u32x4_t*)(qh + 128 * m + 16 * grp);
  const u32x4_t* p1 = (const u32x4_t*)(qh + 128 * m + 64 + 16 * grp);
  c.w[0] = p0[0];
  c.w[1] = p0[1];
  c.w[2] = p1[0];
  c.w[3] = p1[1];
#pragma unroll
  for (int s = 0; s < 2; ++s) c.rope[s] = *(const u32x4_t*)(qh + 512 + 16 * grp + 8 * s);
  return c;
}

// Split of one chunk: the e4m3 hi and lo operands and the lane's E8M0 byte
// of each. `sign` (0 or 0x80008000) is xored into every pair of bf16 values:
// a negative softmax scale is applied as |scale| on -q, which is exact.
__device__ __forceinline__ void split_chunk(const QChunk& c, int grp, uint32_t sign, i32x8_t& fhi, i32x8_t& flo,
                                            uint32_t& sc_hi, uint32_t& sc_lo) {
  const u32x4_t w[4] = {c.w[0] ^ sign, c.w[1] ^ sign, c.w[2] ^ sign, c.w[3] ^ sign};
  float x[32];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[8 * v + 2 * k] = bf16_lo(w[v][k]);
      x[8 * v + 2 * k + 1] = bf16_hi(w[v][k]);
    }
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    m0 = fmaxf(m0, fabsf(x[k]));
    m1 = fmaxf(m1, fabsf(x[16 + k]));
  }
  // The other half of blocks grp/2 and 2 + grp/2 sits in lane group grp ^ 1.
  m0 = fmaxf(m0, __shfl_xor(m0, 16));
  m1 = fmaxf(m1, __shfl_xor(m1, 16));
  const int s0 = e8m0_for_max(m0);   // block grp/2
  const int s1 = e8m0_for_max(m1);   // block 2 + grp/2
  int hi[8], lo[8];
  split16(x, s0, hi, lo);
  split16(x + 16, s1, hi + 4, lo + 4);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    fhi[d] = hi[d];
    flo[d] = lo[d];
  }
  // Block grp's scale: own s0 (grp 0), own s1 (grp 3), else lane group grp ^ 2's.
  const int o0 = __shfl_xor(s0, 32), o1 = __shfl_xor(s1, 32);
  const int sup = grp == 0 ? s0 : grp == 3 ? s1 : grp == 1 ? o0 : o1;
  sc_hi = (uint32_t)sup;
  sc_lo = (uint32_t)max(sup - 4, 0);
}

// LDS staging of the split chunks (in the hand-off area, free until round
// 0): [chunk][hi | lo][lane] 32-byte slots, then [hi | lo][lane] dwords of
// E8M0 bytes (byte m = chunk m). Written and read with inline assembly, so
// that the compiler does not hold them behind the tile loads in flight;
// the writes are complete at the barrier between (see stage_q / fetch_q).
constexpr int kQStage = 4 * 2 * 64 * 32;                   // 16 KB
static_assert(kQStage == 2 * kPairs * 64 * 32, "the q stage fills the hand-off area");

__device__ __forceinline__ void stage_q(uint8_t* stage, uint8_t* stage_sc, int m, int lane, const i32x8_t& hi,
                                        const i32x8_t& lo, uint32_t sc_hi, uint32_t sc_lo) {
  const uint32_t a = lds_addr(stage + (m * 2 * 64 + lane) * 32);
  const u32x4_t h0 = {(uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)hi[2], (uint32_t)hi[3]};
  const u32x4_t h1 = {(uint32_t)hi[4], (uint32_t)hi[5], (uint32_t)hi[6], (uint32_t)hi[7]};
  const u32x4_t l0 = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3]};
  const u32x4_t l1 = {(uint32_t)lo[4], (uint32_t)lo[5], (uint32_t)lo[6], (uint32_t)lo[7]};
  asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:16\n\t"
               "ds_write_b128 %0, %3 offset:2048\n\tds_write_b128 %0, %4 offset:2064"
               ::"v"(a), "v"(h0), "v"(h1), "v"(l0), "v"(l1) : "memory");
  const uint32_t sa = lds_addr(stage_sc + 4 * lane + m);
  asm volatile("ds_write_b8 %0, %1\n\tds_write_b8 %0, %2 offset:256" ::"v"(sa), "v"(sc_hi), "v"(sc_lo)
               : "memory");
}

__device__ __forceinline__ QOperands fetch_q(const uint8_t* stage, const uint8_t* stage_sc, int lane,
                                             const QChunk& own, uint32_t sign) {
  QOperands f;
  u32x4_t r[16];
  const uint32_t a = lds_addr(stage + lane * 32);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // chunk m: hi at m * 4096, lo 2048 further
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * m + 0]) : "v"(a), "i"(m * 4096));
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * m + 1]) : "v"(a), "i"(m * 4096 + 16));
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * m + 2]) : "v"(a), "i"(m * 4096 + 2048));
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * m + 3]) : "v"(a), "i"(m * 4096 + 2064));
  }
  uint32_t sh, sl;
  const uint32_t sa = lds_addr(stage_sc + 4 * lane);
  asm volatile("ds_read_b32 %0, %1" : "=v"(sh) : "v"(sa));
  asm volatile("ds_read_b32 %0, %1 offset:256" : "=v"(sl) : "v"(sa));
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]),
                 "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]), "+v"(r[12]), "+v"(r[13]), "+v"(r[14]),
                 "+v"(r[15]), "+v"(sh), "+v"(sl));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f.hi[m] = i32x8_t{(int)r[4 * m][0], (int)r[4 * m][1], (int)r[4 * m][2], (int)r[4 * m][3],
                      (int)r[4 * m + 1][0], (int)r[4 * m + 1][1], (int)r[4 * m + 1][2], (int)r[4 * m + 1][3]};
    f.lo[m] = i32x8_t{(int)r[4 * m + 2][0], (int)r[4 * m + 2][1], (int)r[4 * m + 2][2], (int)r[4 * m + 2][3],
                      (int)r[4 * m + 3][0], (int)r[4 * m + 3][1], (int)r[4 * m + 3][2], (int)r[4 * m + 3][3]};
  }
  f.sc_hi = sh;
  f.sc_lo = sl;
#pragma unroll
  for (int s = 0; s < 2; ++s) f.rope[s] = __builtin_bit_cast(bf16x8_t, own.rope[s] ^ sign);
  return f;
}

// One 128-dim chunk of S^T: A = 32 fp4 dims of the lane's token row with
// their E8M0 byte, B = the chunk's e4m3 Q part with the scale byte M.
template <int M>
__device__ __forceinline__ f32x4_t mx_chunk(const u32x4_t& k, uint32_t k_scale, const i32x8_t& q,
                                            uint32_t q_scales, f32x4_t acc) {
  const i32x8_t a = {(int32_t)k[0], (int32_t)k[1], (int32_t)k[2], (int32_t)k[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q, acc, 4, 0, 0, (int32_t)k_scale, M,
                                                          (int32_t)q_scales);
}

// S^T = K Q^T for one 16-token sub-tile: returns, for head `col`, the raw
// scores of tokens 16*sub + 4*grp + r (r = 0..3).
template <bool kGather>
__device__ __forceinline__ f32x4_t qk_subtile(const uint8_t* buf, int delta, int sub,
                                              const QOperands& qo, int lane) {
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int row = 16 * sub + col;
  const uint8_t* rp = buf + row * kLdsRow;
  u32x4_t c[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) c[m] = *(const u32x4_t*)(rp + 16 * (4 * m + grp));
  const u32x2_t rope = *(const u32x2_t*)(rp + 256 + 8 * grp);
  const uint8_t* er = scale_row<kGather>(buf, delta, row);
  uint32_t e[5];
#pragma unroll
  for (int m = 0; m < 4; ++m) e[m] = er[4 * m + grp];
  e[4] = er[16 + (grp >> 1)];
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  a0 = mx_chunk<0>(c[0], e[0], qo.hi[0], qo.sc_hi, a0);
  a1 = mx_chunk<0>(c[0], e[0], qo.lo[0], qo.sc_lo, a1);
  a0 = mx_chunk<1>(c[1], e[1], qo.hi[1], qo.sc_hi, a0);
  a1 = mx_chunk<1>(c[1], e[1], qo.lo[1], qo.sc_lo, a1);
  a0 = mx_chunk<2>(c[2], e[2], qo.hi[2], qo.sc_hi, a0);
  a1 = mx_chunk<2>(c[2], e[2], qo.lo[2], qo.sc_lo, a1);
  a0 = mx_chunk<3>(c[3], e[3], qo.hi[3], qo.sc_hi, a0);
  a1 = mx_chunk<3>(c[3], e[3], qo.lo[3], qo.sc_lo, a1);
  const float sr = exp_field(e[4]);
  a0 = mfma(dequant8(rope[0], sr), qo.rope[0], a0);
  a1 = mfma(dequant8(rope[1], sr), qo.rope[1], a1);
  return a0 + a1;
}

// Online-softmax update with the scores of one 32-token tile (s0: tokens
// 4*grp + r of the first sub-tile, s1: of the second, for head `col`):
// returns the tile's hand-off to the P V wave and folds the bf16-rounded
// P into l.
// `csc` >= 0 (a negative scale reaches here as |scale| with q negated).
// `nvalid` = tokens of the tile inside the item (ke - t0, computed as a
// difference so that offsets near 2^31 cannot wrap).
__device__ __forceinline__ TileHandoff softmax_tile(f32x4_t s0, f32x4_t s1, int nvalid,
                                                    SoftmaxState& st, float csc, int lane) {
  const int grp = lane >> 4;
  float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  const bool tail = nvalid < kTile;
  if (tail) {   // tail tile: tokens past the item take no part in the max
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * grp + r >= nvalid) x[r] = kNegInf;
      if (16 + 4 * grp + r >= nvalid) x[4 + r] = kNegInf;
    }
  }
  float mx = max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), fmaxf(x[6], x[7]));
  mx = max_over_groups(mx) * csc;
  const bool need = mx > st.m + kTau;
  TileHandoff h;
  h.alpha = f32x4_t{1.f, 1.f, 1.f, 1.f};
  if (__ballot(need)) {
    const float m_new = need ? mx : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.0f;
    st.m = m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) h.alpha[r] = __shfl(alpha, 4 * grp + r);
    st.l *= h.alpha;
  }
  const float base = st.m;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], csc, -base));
  if (tail) {
    // p = 0 past the item, set after the exponential: with a zero scale the
    // masked -inf * 0 would be NaN
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * grp + r >= nvalid) p[r] = 0.f;
      if (16 + 4 * grp + r >= nvalid) p[4 + r] = 0.f;
    }
  }
  const bf16x8_t pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                       (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
  // l += sum_t P[h][t] of the same bf16-rounded P that multiplies V
  const bf16x8_t ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                         (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  st.l = mfma(pa, ones, st.l);
  h.p = __builtin_bit_cast(u32x4_t, pa);
  return h;
}

// One scale block (32 latent dims) of O += P V: decode the 8 tokens' V bytes
// with their scales and multiply. LB is the block, the reads of block LB + 1
// are issued before this block's wait so that they overlap its decode.
template <int LB>
__device__ __forceinline__ void pv_block(uint32_t tra, uint32_t sca, u32x2_t& v_cur, u32x4_t& s_lo,
                                         u32x4_t& s_hi, const bf16x8_t& pa, f32x4_t (&o)[32]) {
  constexpr int kScStep = kTile * 4;
  u32x2_t v_nx;
  u32x4_t s_nlo, s_nhi;
  if constexpr (LB + 1 < kVBlocks) {
    v_nx = lds_tr8<16 * (LB + 1)>(tra);
    s_nlo = lds_b128<(LB + 1) * kScStep>(sca);
    s_nhi = lds_b128<(LB + 1) * kScStep + 16>(sca);
    asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(v_cur), "+v"(s_lo), "+v"(s_hi));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v_cur), "+v"(s_lo), "+v"(s_hi));
  }
  const uint32_t sv[8] = {s_lo[0], s_lo[1], s_lo[2], s_lo[3], s_hi[0], s_hi[1], s_hi[2], s_hi[3]};
  uint32_t c[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const float scl = __builtin_bit_cast(float, sv[kk]);
    const uint32_t src = kk < 4 ? v_cur[0] : v_cur[1];
    bf16x2_t cv;
    switch (kk & 3) {
      case 0: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 0); break;
      case 1: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 1); break;
      case 2: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 2); break;
      default: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 3); break;
    }
    c[kk] = __builtin_bit_cast(uint32_t, cv);
  }
  // B operands of the block's even (odd) dims: the low (high) halves of the
  // decoded dwords, two tokens per dword
  const u32x4_t be = {__builtin_amdgcn_perm(c[1], c[0], 0x05040100u), __builtin_amdgcn_perm(c[3], c[2], 0x05040100u),
                      __builtin_amdgcn_perm(c[5], c[4], 0x05040100u), __builtin_amdgcn_perm(c[7], c[6], 0x05040100u)};
  const u32x4_t bo = {__builtin_amdgcn_perm(c[1], c[0], 0x07060302u), __builtin_amdgcn_perm(c[3], c[2], 0x07060302u),
                      __builtin_amdgcn_perm(c[5], c[4], 0x07060302u), __builtin_amdgcn_perm(c[7], c[6], 0x07060302u)};
  o[2 * LB] = mfma(pa, __builtin_bit_cast(bf16x8_t, be), o[2 * LB]);
  o[2 * LB + 1] = mfma(pa, __builtin_bit_cast(bf16x8_t, bo), o[2 * LB + 1]);
  if constexpr (LB + 1 < kVBlocks) {
    v_cur = v_nx;
    s_lo = s_nlo;
    s_hi = s_nhi;
    pv_block<LB + 1>(tra, sca, v_cur, s_lo, s_hi, pa, o);
  }
}

// O += P V over all 512 latent dims for one tile (rows in `buf`, formatted
// scales in `fmt`), after rescaling O by the hand-off's alpha.
__device__ __forceinline__ void pv_tile(const uint8_t* buf, const uint8_t* fmt, const TileHandoff& h,
                                        f32x4_t (&o)[32], int lane) {
  const int col = lane & 15;
  const int grp = lane >> 4;
  const bool resc = h.alpha[0] != 1.f || h.alpha[1] != 1.f || h.alpha[2] != 1.f || h.alpha[3] != 1.f;
  if (__ballot(resc)) {
#pragma unroll
    for (int n = 0; n < 32; ++n) o[n] *= h.alpha;
  }
  // A operand: P of head `col` at the 8 tokens of lane group `grp`, in the
  // order of the V rows below (K = the tile's 32 tokens).
  const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, h.p);
  // lane (col, grp) supplies row k = col/2 of its group's 8 tokens, bytes
  // 8*(col&1).. of a 16-byte column block; it receives byte (16B + col) of
  // all 8 tokens, in the order of the formatted scales.
  const int k = col >> 1;
  const int trow = 4 * grp + (k & 3) + 16 * (k >> 2);
  const uint32_t tra = lds_addr(buf + trow * kLdsRow + 8 * (col & 1));
  const uint32_t sca = lds_addr(fmt + 32 * grp);
  u32x2_t v_cur = lds_tr8<0>(tra);
  u32x4_t s_lo = lds_b128<0>(sca), s_hi = lds_b128<16>(sca);
  pv_block<0>(tra, sca, v_cur, s_lo, s_hi, pa, o);
}

// kGather: rows listed through kv_indices (kPages: as a page table). kStarts
// (contiguous rows only): sequence b starts at row kv_start[b], so that
// several entries can share rows. Each mode is its own instantiation; the
// plain contiguous kernel carries none of the others' code.
// One plan item: sequence, token range, partial index (-1: direct output).
struct __attribute__((aligned(16))) ItemWords {
  int32_t b, kb, ke, dest;
};
typedef const __attribute__((address_space(4))) int32_t ConstI32;

template <bool kGather, bool kPages, bool kStarts = false>
__global__ void __launch_bounds__(kThreads, 1)
mla_decode_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                  const uint8_t* __restrict__ sc, const int32_t* __restrict__ kv_indptr,
                  const int32_t* __restrict__ kv_indices, const int32_t* __restrict__ page_indptr,
                  int page_size, const int32_t* __restrict__ kv_start, uint16_t* __restrict__ out,
                  const int32_t* __restrict__ plan, float* __restrict__ part_lse, float* __restrict__ part_out,
                  float csc) {
  using L = Lds<kGather>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kTotal];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool scorer = (wave >> 2) != 0;   // else the pair's P V wave
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // Workgroups are dealt to the 8 XCDs in turn. When entries share rows
  // (kv_start), consecutive slots -- the query groups of one sequence --
  // go to workgroups of one XCD, so that its L2 serves the repeated reads.
  const bool xcd_order = kStarts && (gridDim.x & 7) == 0;
  const int first_slot = xcd_order ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                                   : (int)blockIdx.x;
  // The header words and the first slot's bounds in slot_indptr (which
  // both planners place right after the header, and which has an entry for
  // every launched workgroup) are read in one batch, before the check: a
  // memory latency each saved on the way to the first tile.
  const int32_t* slot_indptr = plan + MLA_PLAN_HEADER_WORDS;
  const int magic = plan[kPwMagic];
  const int version = plan[kPwVersion];
  const int num_slots = plan[kPwNumSlots];
  const int off_items = plan[kPwOffItems];
  int i_begin = slot_indptr[first_slot];
  int i_end = slot_indptr[first_slot + 1];
  // The first slot's first item, read in the same batch from where it sits
  // when the items start right after slot_indptr of a launch-sized plan and
  // every slot before this one holds one item (item index = slot index).
  // It is used only when the header and slot_indptr confirm both, else the
  // item is loaded after them. The words read lie inside the plan in every
  // case: a plan has at least the launched number of slots, its items start
  // at or after this offset, and it has at least one item per slot.
  const int spec_off = (MLA_PLAN_HEADER_WORDS + (int)gridDim.x + 1 + 3) & ~3;
  const ItemWords spec = *(const ItemWords*)(plan + spec_off + 4 * first_slot);
  // (the compiler would otherwise load each only where it is first used,
  // one latency after another; the kernel arguments are fetched here too)
  asm volatile("" ::"s"(num_slots), "s"(off_items), "s"(i_begin), "s"(i_end), "s"(spec.b), "s"(spec.kb),
               "s"(spec.ke), "s"(spec.dest), "s"(q), "s"(kv), "s"(sc), "s"(kv_indptr), "s"(out));
  // Only words written by a planner are followed: a workspace whose header
  // is not a plan of this version (never planned, overwritten, or an
  // empty device plan) leaves the output untouched.
  if (magic != MLA_PLAN_MAGIC || version != MLA_PLAN_VERSION) return;
  // A negative scale is applied as |scale| on -q (exact), so the running
  // max below is a max of the scaled scores whatever the scale's sign.
  const uint32_t qsign = csc < 0.f ? 0x80008000u : 0u;
  csc = fabsf(csc);

  const int32_t* items = plan + off_items;
  // kv_indptr is not written while the kernel runs: read it through the
  // constant address space, so that its words come by scalar loads
  const ConstI32* kv_indptr_s = (const ConstI32*)kv_indptr;
  uint8_t* ring = lds + pair * L::kPair;
  TileHandoff* hand = (TileHandoff*)(lds + L::kXchg) + pair * 64 + lane;  // + parity * kPairs * 64
  uint8_t* fmt_pair = lds + L::kFmt + pair * kFmtTile;  // + parity * kPairs * kFmtTile
  // The scorer's results gate the next round of both waves: it gets issue
  // priority over the P V wave on the shared SIMD.
  if (scorer) __builtin_amdgcn_s_setprio(1);

  for (int slot = first_slot; slot < num_slots; slot += gridDim.x) {
    if (slot != first_slot) {
      i_begin = slot_indptr[slot];
      i_end = slot_indptr[slot + 1];
    }
    for (int it = i_begin; it < i_end; ++it) {
      const ItemWords iw = slot == first_slot && it == first_slot && off_items == spec_off
                               ? spec : *(const ItemWords*)(items + 4 * it);
      const int b = iw.b;
      const int dest = iw.dest;
      // first entry of the sequence in kv_indices: its page list, or its rows
      const int ibase = kPages ? page_indptr[b] : 0;   // the sequence's first page entry
      // The item's rows, clamped to the sequence (a plan made for other
      // offsets reads nothing outside it). Each role takes them on its own
      // path, the scorer after it has requested q (scalar loads here; the q
      // loads are vector loads), so that q flies while they are waited for.
      struct Range {
        int seq_lo, kb, ke, rounds, ntiles, t_first;
      };
      auto item_range = [&]() {
        Range r;
        r.seq_lo = kv_indptr_s[b];
        r.kb = max(iw.kb, r.seq_lo);
        r.ke = min(iw.ke, kv_indptr_s[b + 1]);
        // counts from differences, so that offsets near 2^31 - 1 cannot
        // wrap; a tile start is only formed for tiles inside the item
        const int len = r.ke - r.kb;
        r.rounds = len > 0 ? (len - 1) / kTileStride + 1 : 0;
        const int rel_first = kTile * pair;
        r.ntiles = rel_first < len ? (len - rel_first - 1) / kTileStride + 1 : 0;
        r.t_first = r.ntiles > 0 ? r.kb + rel_first : r.kb;
        return r;
      };

      // The pair splits a tile's work by role, each wave on its own loop
      // (both pass the same workgroup barriers, one per round):
      //  * the scorer stages tiles (one in flight), computes S for the whole
      //    tile, runs the softmax and formats the V scales;
      //  * the P V wave accumulates O over all 512 dims one round later.
      // Round i: scores of tile i, P V of tile i - 1.
      // Each role's state lives only on its own path (it is written to LDS
      // for the merge before the paths join).
      f32x4_t* frag = (f32x4_t*)lds;
      float* stats = (float*)(lds + kMergeFrag);
      if (scorer) {
        SoftmaxState st;
        st.l = f32x4_t{0.f, 0.f, 0.f, 0.f};
        st.m = kMInit;
        const QChunk qc = load_q_chunk(q + ((size_t)b * kHeads + col) * kQkDim, pair, grp);
        const Range rg = item_range();
        const int seq_lo = rg.seq_lo, ke = rg.ke, rounds = rg.rounds, ntiles = rg.ntiles, t_first = rg.t_first;
        // contiguous rows: with kv_start the sequence's tokens are the rows
        // from kv_start[b] on (several sequences may share them); the tile
        // code keeps kv_indptr positions and reads through shifted bases
        const uint8_t* kv_b = kv;
        const uint8_t* sc_b = sc;
        if (kStarts) {
          const ptrdiff_t shift = (ptrdiff_t)kv_start[b] - seq_lo;
          kv_b += shift * kRowBytes;
          sc_b += shift * kBlocks;
        }
        PageRows pages = {0u, 0u};   // page tables: the entries of the next tile to stage
        __syncthreads();  // LDS of the previous item's merge is free again
        // Contiguous rows: q's loads went out before the bounds were waited
        // for and have landed by now. Taking them here, before tile 0 is
        // requested, lets the split below run while the tile flies (a wait
        // for q after the tile's loads would also wait for the tile).
        if constexpr (!kGather) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        if (ntiles > 0) {
          if constexpr (kPages) {
            // rows of tile 0, then its staging; the pages of tile 1 fly
            store_page_rows(ring, load_pages(kv_indices, ibase, t_first - seq_lo, ke - t_first, page_size, lane),
                            page_size, lane);
            if (ntiles > 1)
              pages = load_pages(kv_indices, ibase, t_first + kTileStride - seq_lo, ke - t_first - kTileStride,
                                 page_size, lane);
            stage_gather(ring, kv, sc, ke - t_first, lane);
          } else if constexpr (kGather) {
            // row indices of the first two tiles, then tile 0 from them
            stage_idx(ring, kv_indices, t_first, ke - t_first, lane);
            if (ntiles > 1)
              stage_idx(ring + L::kBuf, kv_indices, t_first + kTileStride, ke - t_first - kTileStride, lane);
            wait_dma();
            stage_gather(ring, kv, sc, ke - t_first, lane);
          } else {
            stage_dma(ring, kv_b, sc_b, t_first, ke - t_first, lane);
          }
        }
        {
          i32x8_t qhi, qlo;
          uint32_t qsh, qsl;
          split_chunk(qc, grp, qsign, qhi, qlo, qsh, qsl);
          stage_q(lds + L::kXchg, lds + L::kFmt, pair, lane, qhi, qlo, qsh, qsl);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();  // all four chunks staged
        const QOperands qo = fetch_q(lds + L::kXchg, lds + L::kFmt, lane, qc, qsign);
        for (int i = 0; i <= rounds; ++i) {
          const bool qk_on = i < ntiles;
          if (qk_on) wait_dma();
          __syncthreads();  // tile i landed; tile i-2 fully consumed; hand-off of i-1 visible
          if (i + 1 < ntiles) {
            const int tn = t_first + (i + 1) * kTileStride;
            if constexpr (kPages) {
              // tile i + 1's rows from the pages loaded a round ago (the
              // round's wait above drained them too), then the pages of i + 2
              uint8_t* bn = ring + ((i + 1) % kNumBuf) * L::kBuf;
              store_page_rows(bn, pages, page_size, lane);
              stage_gather(bn, kv, sc, ke - tn, lane);
              if (i + 2 < ntiles)
                pages = load_pages(kv_indices, ibase, tn + kTileStride - seq_lo, ke - tn - kTileStride, page_size,
                                   lane);
            } else if constexpr (kGather) {
              // tile i + 1 from the indices staged a round ago; the indices
              // of tile i + 2 go to the slot of the buffer it will use (the
              // P V wave reads only that buffer's rows this round)
              stage_gather(ring + ((i + 1) % kNumBuf) * L::kBuf, kv, sc, ke - tn, lane);
              if (i + 2 < ntiles)
                stage_idx(ring + ((i + 2) % kNumBuf) * L::kBuf, kv_indices, tn + kTileStride,
                          ke - tn - kTileStride, lane);
            } else {
              stage_dma(ring + ((i + 1) % kNumBuf) * L::kBuf, kv_b, sc_b, tn, ke - tn, lane);
            }
          }
          if (qk_on) {
            const int tq = t_first + i * kTileStride;
            const uint8_t* bq = ring + (i % kNumBuf) * L::kBuf;
            const int dq = kGather ? (int)((uintptr_t)sc & 15) : raw_delta(sc_b, tq);
            const f32x4_t s0 = qk_subtile<kGather>(bq, dq, 0, qo, lane);
            const f32x4_t s1 = qk_subtile<kGather>(bq, dq, 1, qo, lane);
            hand[(i & 1) * (kPairs * 64)] = softmax_tile(s0, s1, ke - tq, st, csc, lane);
            uint8_t* fm = fmt_pair + (i & 1) * (kPairs * kFmtTile);
            format_scales<kGather>(bq, fm, dq, ke - tq, lane);
            format_scales<kGather>(bq, fm, dq, ke - tq, 64 + lane);
          }
        }
        __syncthreads();  // all rounds done: the ring area is free for the merge
        if (grp == 0) stats[(2 * pair) * kHeads + col] = st.m;
        if (col == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) stats[(2 * pair + 1) * kHeads + 4 * grp + r] = st.l[r];
        }
      } else {
        const Range rg = item_range();
        const int rounds = rg.rounds, ntiles = rg.ntiles;
        f32x4_t o[32];
#pragma unroll
        for (int n = 0; n < 32; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        __syncthreads();  // (the scorers stage q between the two)
        for (int i = 0; i <= rounds; ++i) {
          __syncthreads();
          if (i >= 1 && i - 1 < ntiles) {
            const TileHandoff h = hand[((i - 1) & 1) * (kPairs * 64)];
            pv_tile(ring + ((i - 1) % kNumBuf) * L::kBuf, fmt_pair + ((i - 1) & 1) * (kPairs * kFmtTile),
                    h, o, lane);
          }
        }
        __syncthreads();
#pragma unroll
        for (int f = 0; f < 32; ++f) frag[(pair * 32 + f) * 64 + lane] = o[f];
      }

      // ---- merge the 4 pairs' states ----
      __syncthreads();

      float wgt[4][kPairs];
      float inv[4];
      float lse[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        float mw[kPairs], lw[kPairs];
        float mmax = kNegInf;
#pragma unroll
        for (int w = 0; w < kPairs; ++w) {
          mw[w] = stats[(2 * w) * kHeads + h];
          lw[w] = stats[(2 * w + 1) * kHeads + h];
          if (lw[w] != 0.f) mmax = fmaxf(mmax, mw[w]);
        }
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kPairs; ++w) {
          wgt[r][w] = lw[w] != 0.f ? __builtin_amdgcn_exp2f(mw[w] - mmax) : 0.f;
          lsum += wgt[r][w] * lw[w];
        }
        inv[r] = lsum != 0.f ? 1.0f / lsum : 0.f;
        lse[r] = lsum != 0.f ? mmax + __builtin_amdgcn_logf(lsum) : kNegInf;
      }
      // wave w writes scale blocks 2w, 2w+1 (both dim parities)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int blk = 2 * wave + bb;
        f32x4_t ev = {0.f, 0.f, 0.f, 0.f}, od = ev;
#pragma unroll
        for (int w = 0; w < kPairs; ++w) {
          const f32x4_t fe = frag[(w * 32 + 2 * blk) * 64 + lane];
          const f32x4_t fo = frag[(w * 32 + 2 * blk + 1) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ev[r] += wgt[r][w] * fe[r];
            od[r] += wgt[r][w] * fo[r];
          }
        }
        const int d = 32 * blk + 2 * col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 4 * grp + r;
          const float re = ev[r] * inv[r], ro = od[r] * inv[r];
          if (dest < 0) {
            *(uint32_t*)(out + ((size_t)b * kHeads + h) * kVDim + d) = pack2(re, ro);
          } else {
            *(f32x2_t*)(part_out + ((size_t)dest * kHeads + h) * kVDim + d) = f32x2_t{re, ro};
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

// LSE-weighted merge of the partials of one sequence (or zero fill of an
// empty one), for plans with long splits (many partials per sequence):
// out = sum_p 2^(lse_p - M) O_p / sum_p 2^(lse_p - M) with M = max_p lse_p
// over non-empty partials. One workgroup per (reduce entry, head, 32-dim
// slice), so that a single long sequence still spreads its partials' reads
// over 256 workgroups. Its 16 waves x 4 lane groups are 64 streams, stream s
// taking partials s, s + 64, ...; a lane group's 16 lanes cover the slice's
// 32 dims two each. Every stream keeps a running max and rescales its sums
// when it rises; the streams are combined by shuffles within the wave, then
// through LDS across the waves.
constexpr int kReduceWaves = 16;
constexpr int kReduceThreads = 64 * kReduceWaves;
constexpr int kReduceSplit = 16;                     // 32-dim slices per head
constexpr int kReduceStreams = 4 * kReduceWaves;     // 4 lane groups per wave
static_assert(kVDim / kReduceSplit == 2 * 16, "reduce: a lane group covers one slice, two dims per lane");

// (m, s, a) <- the merge of two running states (m = -inf: empty)
__device__ __forceinline__ void merge_state(float& m, float& s, f32x2_t& a, float m2, float s2, f32x2_t a2) {
  const float mm = fmaxf(m, m2);
  const float f1 = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mm);
  const float f2 = m2 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
  s = s * f1 + s2 * f2;
  a = a * f1 + a2 * f2;
  m = mm;
}

__global__ void __launch_bounds__(kReduceThreads)
mla_reduce_kernel(const int32_t* __restrict__ plan, const float* __restrict__ part_lse,
                  const float* __restrict__ part_out, uint16_t* __restrict__ out) {
  __shared__ f32x2_t acc_s[kReduceWaves][16];
  __shared__ float wsum_s[kReduceWaves];
  __shared__ float max_s[kReduceWaves];
  // header words in one batch; a plan built on the GPU is launched for its
  // bound on the entry count
  const int magic = plan[kPwMagic];
  const int version = plan[kPwVersion];
  const int num_reduce = plan[kPwNumReduce];
  const int off_reduce = plan[kPwOffReduce];
  asm volatile("" ::"s"(num_reduce), "s"(off_reduce), "s"(part_lse), "s"(part_out), "s"(out));
  if (magic != MLA_PLAN_MAGIC || version != MLA_PLAN_VERSION) return;
  if ((int)blockIdx.x >= num_reduce) return;
  const int32_t* ent = plan + off_reduce + 4 * blockIdx.x;
  const int b = ent[0];
  const int first = ent[1];
  const int cnt = ent[2];
  const int h = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int d = (kVDim / kReduceSplit) * blockIdx.z + 2 * l16;
  uint32_t* dst = (uint32_t*)(out + ((size_t)b * kHeads + h) * kVDim + d);
  if (cnt == 0) {
    if (wave == 0 && lane < 16) *dst = 0u;
    return;
  }
  constexpr int kUnroll = 4;
  float m = kNegInf;
  f32x2_t acc = {0.f, 0.f};
  float wsum = 0.f;
  const int stream = 4 * wave + (lane >> 4);
  for (int i0 = stream; i0 < cnt; i0 += kUnroll * kReduceStreams) {
    float v[kUnroll];
    f32x2_t o[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = min(i0 + u * kReduceStreams, cnt - 1);
      v[u] = part_lse[(size_t)(first + i) * kHeads + h];
      o[u] = *(const f32x2_t*)(part_out + ((size_t)(first + i) * kHeads + h) * kVDim + d);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (i0 + u * kReduceStreams < cnt && v[u] != kNegInf) {
        const float m_new = fmaxf(m, v[u]);
        const float keep = __builtin_amdgcn_exp2f(m - m_new);   // 0 while m is -inf
        const float w = __builtin_amdgcn_exp2f(v[u] - m_new);
        wsum = wsum * keep + w;
        acc = acc * keep + w * o[u];
        m = m_new;
      }
    }
  }
  // the wave's 4 lane groups (same dims, other partials)
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(wsum, off);
    const f32x2_t a2 = {__shfl_xor(acc[0], off), __shfl_xor(acc[1], off)};
    merge_state(m, wsum, acc, m2, s2, a2);
  }
  if (lane < 16) acc_s[wave][lane] = acc;
  if (lane == 0) {
    wsum_s[wave] = wsum;
    max_s[wave] = m;
  }
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kReduceWaves; ++w) mm = fmaxf(mm, max_s[w]);
    f32x2_t tot = {0.f, 0.f};
    float ws = 0.f;
#pragma unroll
    for (int w = 0; w < kReduceWaves; ++w) {
      if (max_s[w] != kNegInf) {
        const float sc = __builtin_amdgcn_exp2f(max_s[w] - mm);
        tot += sc * acc_s[w][lane];
        ws += sc * wsum_s[w];
      }
    }
    const float inv = ws != 0.f ? 1.0f / ws : 0.f;
    *dst = pack2(tot[0] * inv, tot[1] * inv);
  }
}

// The same merge for plans whose split sequences have few partials each
// (many sequences, a handful of splits): one 64-thread workgroup per
// (reduce entry, head), each lane covering 8 consecutive output dims, so a
// workgroup reads its partials with 16-byte loads and no LDS round. The
// wide kernel above spreads one sequence's partials over 16 waves, which a
// long split needs but which leaves most waves idle here.
constexpr int kNarrowThreads = 64;
static_assert(kVDim == 8 * kNarrowThreads, "narrow reduce: a lane covers 8 dims");

__global__ void __launch_bounds__(kNarrowThreads)
mla_reduce_narrow_kernel(const int32_t* __restrict__ plan, const float* __restrict__ part_lse,
                         const float* __restrict__ part_out, uint16_t* __restrict__ out) {
  // header words in one batch (the compiler would fetch each after the
  // previous check), then the entry
  const int magic = plan[kPwMagic];
  const int version = plan[kPwVersion];
  const int num_reduce = plan[kPwNumReduce];
  const int off_reduce = plan[kPwOffReduce];
  asm volatile("" ::"s"(num_reduce), "s"(off_reduce), "s"(part_lse), "s"(part_out), "s"(out));
  if (magic != MLA_PLAN_MAGIC || version != MLA_PLAN_VERSION) return;
  if ((int)blockIdx.x >= num_reduce) return;
  const int32_t* ent = plan + off_reduce + 4 * blockIdx.x;
  const int b = ent[0];
  const int first = ent[1];
  const int cnt = ent[2];
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int d = 8 * lane;
  u32x4_t* dst = (u32x4_t*)(out + ((size_t)b * kHeads + h) * kVDim + d);
  if (cnt == 0) {
    *dst = u32x4_t{0u, 0u, 0u, 0u};
    return;
  }
  // partials in order, four at a time with all their loads in flight; the
  // first four go out together with the LSE loads of the max
  constexpr int kUnroll = 4;
  float v[kUnroll];
  f32x4_t o0[kUnroll], o1[kUnroll];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = min(i0 + u, cnt - 1);
      v[u] = part_lse[(size_t)(first + i) * kHeads + h];
      const f32x4_t* src = (const f32x4_t*)(part_out + ((size_t)(first + i) * kHeads + h) * kVDim + d);
      o0[u] = src[0];
      o1[u] = src[1];
    }
  };
  load_batch(0);
  float m = kNegInf;
  for (int i = lane; i < cnt; i += kNarrowThreads) {
    const float x = part_lse[(size_t)(first + i) * kHeads + h];
    if (x != kNegInf) m = fmaxf(m, x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  float wsum = 0.f;
  for (int i0 = 0; i0 < cnt; i0 += kUnroll) {
    if (i0 > 0) load_batch(i0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (i0 + u < cnt && v[u] != kNegInf) {
        const float w = __builtin_amdgcn_exp2f(v[u] - m);
        wsum += w;
        a0 += w * o0[u];
        a1 += w * o1[u];
      }
    }
  }
  const float inv = wsum != 0.f ? 1.0f / wsum : 0.f;
  *dst = u32x4_t{pack2(a0[0] * inv, a0[1] * inv), pack2(a0[2] * inv, a0[3] * inv),
                 pack2(a1[0] * inv, a1[1] * inv), pack2(a1[2] * inv, a1[3] * inv)};
}

}  // namespace

size_t decode_lds_bytes() { return (size_t)Lds<true>::kTotal; }

int launch_decode(const DecodeArgs& a, void* stream) {
  if (a.num_slots <= 0 || a.grid <= 0) return (int)hipSuccess;
  if (a.kv_indices != nullptr) {
    if (a.page_indptr != nullptr)
      hipLaunchKernelGGL((mla_decode_kernel<true, true>), dim3(a.grid), dim3(kThreads), 0, (hipStream_t)stream,
                         (const uint16_t*)a.q, a.kv_packed, a.kv_scale, a.kv_indptr, a.kv_indices,
                         a.page_indptr, a.page_size, (const int32_t*)nullptr, (uint16_t*)a.out, a.plan,
                         a.part_lse, a.part_out, a.score_scale_log2);
    else
      hipLaunchKernelGGL((mla_decode_kernel<true, false>), dim3(a.grid), dim3(kThreads), 0,
                         (hipStream_t)stream, (const uint16_t*)a.q, a.kv_packed, a.kv_scale, a.kv_indptr,
                         a.kv_indices, (const int32_t*)nullptr, 1, (const int32_t*)nullptr, (uint16_t*)a.out,
                         a.plan, a.part_lse, a.part_out, a.score_scale_log2);
  } else {
    if (a.kv_start != nullptr)
      hipLaunchKernelGGL((mla_decode_kernel<false, false, true>), dim3(a.grid), dim3(kThreads), 0,
                         (hipStream_t)stream, (const uint16_t*)a.q, a.kv_packed, a.kv_scale, a.kv_indptr,
                         (const int32_t*)nullptr, (const int32_t*)nullptr, 1, a.kv_start, (uint16_t*)a.out, a.plan,
                         a.part_lse, a.part_out, a.score_scale_log2);
    else
      hipLaunchKernelGGL((mla_decode_kernel<false, false>), dim3(a.grid), dim3(kThreads), 0, (hipStream_t)stream,
                         (const uint16_t*)a.q, a.kv_packed, a.kv_scale, a.kv_indptr, (const int32_t*)nullptr,
                         (const int32_t*)nullptr, 1, (const int32_t*)nullptr, (uint16_t*)a.out, a.plan,
                         a.part_lse, a.part_out, a.score_scale_log2);
  }
  return (int)hipGetLastError();
}

int launch_reduce(const DecodeArgs& a, void* stream) {
  if (a.num_reduce <= 0) return (int)hipSuccess;
  if (a.wide_reduce) {
    hipLaunchKernelGGL(mla_reduce_kernel, dim3(a.num_reduce, kHeads, kReduceSplit), dim3(kReduceThreads), 0,
                       (hipStream_t)stream, a.plan, a.part_lse, a.part_out, (uint16_t*)a.out);
  } else {
    hipLaunchKernelGGL(mla_reduce_narrow_kernel, dim3(a.num_reduce, kHeads), dim3(kNarrowThreads), 0,
                       (hipStream_t)stream, a.plan, a.part_lse, a.part_out, (uint16_t*)a.out);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
