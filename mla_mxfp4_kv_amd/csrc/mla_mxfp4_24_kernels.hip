// HIP kernel for absorbed-MLA decode over the 24-scale MXFP4 cache on gfx950
// (MI355X): the same packed rows as the 18-scale layout (288 bytes, element
// 2j in the low nibble of byte j, e2m1 codes) with 24 E8M0 bytes per token,
// byte k scaling the 24 elements 24k .. 24k+23 (packed bytes 12k .. 12k+11)
// -- the layout of page "kernelbot-amd-mixed-mla-717900" (mxfp4 layout
// comment block, Triton stage-1 loads). What is computed is unchanged
// (page "kernelbot-amd-mixed-mla-676098", _naive_fallback): softmax(sm_scale
// * q . K) V per sequence and head, V the first 512 dequantised elements.
// Plan, partials and reduce are those of the 18-scale decode.
//
// Structure: the one of the 18-scale kernel (mla_kernels.hip): one workgroup
// of 8 waves per CU, persistent over the planner's slots; 32-token tiles
// dealt round-robin to 4 wave pairs, each pair sharing a SIMD and an LDS
// ring of three tile buffers (packed rows as in memory plus the 16-byte
// chunks covering the tile's scale rows, staged by direct global->LDS
// loads, one tile in flight); in each pair a scorer wave computes S, the
// softmax and the formatted V scales, and a P V wave accumulates O one
// round later. What the 24-element blocks change:
//  * QK^T runs entirely on v_mfma_scale_f32_16x16x128_f8f6f4 with every
//    24-element block padded to one 32-element MX block: the 576 dims are
//    24 blocks, six 128-wide steps (rope included). Lane group g of the fp4
//    A operand holds block 4m + g of step m -- its 12 packed bytes and four
//    zero bytes -- with that block's E8M0 byte as its scale; q is split
//    exactly into e4m3 hi + lo per padded block (zero in the padding), so no
//    K element is decoded for the scores;
//  * P V decodes V with the scale of block (32B + 2 col) / 24 for the two
//    dims a lane holds in 32-dim output block B: within one output block
//    the lanes split between two scale blocks at col 12, 8 or 4 (B mod 3 =
//    0, 1, 2), so each lane keeps three addresses into the tile's
//    formatted scale table ([block][position], 22 blocks hold a V dim).
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
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
#define MLA_LDS __attribute__((address_space(3)))

constexpr int kHeads = MLA_NUM_HEADS;
constexpr int kQkDim = MLA_QK_DIM;
constexpr int kVDim = MLA_V_DIM;
constexpr int kRowBytes = MLA_PACKED_BYTES;        // 288
constexpr int kSc = MLA_SCALES_PER_TOKEN_24;       // 24 scale bytes per token
constexpr int kBlk = MLA_SCALE_BLOCK_24;           // 24 elements per scale block
constexpr int kSteps = kQkDim / (4 * kBlk);        // 6 MX steps of 4 padded blocks
constexpr int kWaves = 8;                          // 4 pairs x 2 roles, 2 waves per SIMD
constexpr int kPairs = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;
constexpr int kTileStride = kPairs * kTile;
constexpr int kNumBuf = 3;
constexpr int kRowDma = kTile * kRowBytes / 1024;  // 9 DMA instructions of 1 KB
constexpr int kLdsRaw = kTile * kRowBytes;         // scale chunks after the packed rows
constexpr int kRawChunks = (kTile * kSc) / 16 + 1; // 49 chunks cover 768 bytes at an 8-byte offset
constexpr int kLdsBuf = kLdsRaw + kRawChunks * 16 + 48;   // 10048 (multiple of 64)
constexpr int kLdsPair = kNumBuf * kLdsBuf;
constexpr int kVBlocks = kVDim / 32;               // 16 output blocks of 32 dims
constexpr int kVScaleBlocks = (kVDim + kBlk - 1) / kBlk;  // 22 scale blocks hold a V dim
constexpr int kFmtTile = kVScaleBlocks * kTile * 4;       // [block][position] exponent dwords
constexpr int kLdsFmt = kPairs * kLdsPair;
constexpr int kLdsXchg = kLdsFmt + 2 * kPairs * kFmtTile;
constexpr int kLdsMain = kLdsXchg + 2 * kPairs * 64 * 32;
constexpr int kMergeFrag = kPairs * 32 * 64 * 16;
constexpr int kMergeBytes = kMergeFrag + kPairs * 2 * kHeads * 4;
constexpr int kLdsTotal = kLdsMain > kMergeBytes ? kLdsMain : kMergeBytes;
constexpr float kTau = 8.0f;
constexpr int kStream = 2;                         // non-temporal tile loads
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1.0e30f;
// q staging (before the first round): [step][hi | lo][lane] 32-byte slots,
// then [hi | lo][lane] 8-byte rows of E8M0 bytes (byte m = step m), in the
// V-scale and hand-off areas
constexpr int kQStage = kSteps * 2 * 64 * 32;      // 24 KB
constexpr int kQStageSc = kQStage + 2 * 64 * 8;

static_assert(kLdsTotal <= 160 * 1024, "LDS budget of one gfx950 CU");
static_assert(kLdsBuf % 64 == 0, "buffers stay 64-byte aligned");
static_assert(kSteps == 6 && kQkDim == kSteps * 4 * kBlk, "six steps of four 24-element blocks");
static_assert(kQStageSc <= kLdsMain - kLdsFmt, "the q stage fits the V-scale and hand-off areas");

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS uint8_t*)p;
}

// Offset of a tile's first scale byte inside its 16-byte chunk (0 or 8:
// scale rows are 8-byte aligned).
__device__ __forceinline__ int raw_delta(const uint8_t* sc, int t0) {
  return (int)((uintptr_t)(sc + (size_t)t0 * kSc) & 15);
}

// Stage the 32-token tile starting at token t0 (`nvalid` tokens of it inside
// the item): the packed rows as one contiguous copy (slots past the last
// valid row repeat its last 16 bytes), then the 16-byte chunks that cover
// the tile's scale rows, so that scale byte (row, k) lands at
// buf + kLdsRaw + delta + 24 row + k. Issued by the pair's scorer.
__device__ __forceinline__ void stage_dma(uint8_t* buf, const uint8_t* __restrict__ kv,
                                          const uint8_t* __restrict__ sc, int t0, int nvalid, int lane) {
  t0 = __builtin_amdgcn_readfirstlane(t0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const uint8_t* kv_t = kv + (size_t)t0 * kRowBytes;
  const uint32_t lane_off = 16 * lane;
  if (nvalid >= kTile) {
#pragma unroll
    for (int i = 0; i < kRowDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(kv_t + 1024 * i + lane_off), (MLA_LDS void*)(buf + 1024 * i),
                                       16, 0, kStream);
  } else {
    const uint32_t last = (uint32_t)(nvalid * kRowBytes - 16);
#pragma unroll
    for (int i = 0; i < kRowDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(kv_t + min(1024 * i + lane_off, last)),
                                       (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  }
  const uintptr_t first = (uintptr_t)(sc + (size_t)t0 * kSc);
  const uintptr_t last_chunk = (first + (uintptr_t)(kSc * min(nvalid, kTile)) - 1) & ~(uintptr_t)15;
  const uintptr_t src = min((first & ~(uintptr_t)15) + lane_off, last_chunk);
  if (lane < kRawChunks)
    __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(buf + kLdsRaw), 16, 0, kStream);
}

// Wait for this wave's share of the DMA in flight (vector memory operations
// complete in order); the memory clobber keeps later LDS reads below it.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Rewrite the V scales of a landed tile as exponent-field dwords (e << 23,
// the converter's scale operand) into `fmt` ([block][position], the
// positions in the order lane group g holds its 8 probabilities: 8g + j is
// token 4g + j of the first sub-tile for j < 4, token 16 + 4g + j - 4 of the
// second for j >= 4). `l` (0..175) picks one block and four positions; rows
// at or past `nvalid` get scale 1 (their p is 0).
__device__ __forceinline__ void format_scales(const uint8_t* buf, uint8_t* fmt, int delta, int nvalid, int l) {
  const int blk = l >> 3;
  const int pg = l & 7;
  const int row0 = 16 * (pg & 1) + 4 * (pg >> 1);
  const uint8_t* raw = buf + kLdsRaw + delta + blk;
  u32x4_t v;
  if (nvalid >= kTile) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (uint32_t)raw[kSc * (row0 + j)] << 23;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = raw[kSc * (row0 + j)];
      v[j] = row0 + j < nvalid ? e << 23 : 127u << 23;
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

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

struct SoftmaxState {
  f32x4_t l;         // denominator of heads 4*grp + r (C layout, any column)
  float m;           // running max (base-2 scaled scores) of head `col`
};

// P of one tile in the A-operand layout of the bf16 MFMA and the factor that
// rescales O's rows before the tile is added.
struct TileHandoff {
  u32x4_t p;
  f32x4_t alpha;
};

__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max over lanes h, h+16, h+32, h+48; the swap results are copied to
// scalars before their bit casts (a bit cast of an element of the builtin's
// two-element result reads element 0).
__device__ __forceinline__ float max_over_groups(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float m1 = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t u1 = __builtin_bit_cast(uint32_t, m1);
  const auto c = __builtin_amdgcn_permlane16_swap(u1, u1, false, false);
  const uint32_t c0 = c[0], c1 = c[1];
  return fmaxf(__builtin_bit_cast(float, c0), __builtin_bit_cast(float, c1));
}

// q in the B-operand form of the six MX steps (lane: head `col`, lane group
// `grp`). Step m covers padded blocks 4m .. 4m + 3 (K element 32 i + j of the
// step is element j of block 4m + i, zero for j >= 24). The matrix core pairs
// A lane group g (padded block 4m + g) with B values such that B lane group
// g' holds K elements 16g' .. 16g' + 15 and 64 + 16g' .. 64 + 16g' + 15, and
// B's scale from lane group g' applies to K block g'; so a lane splits its
// two 16-value halves (halves of blocks g'/2 and 2 + g'/2) with those
// blocks' scales and supplies block g''s scale byte. Each bf16 q is split
// exactly into hi * 2^(sh-127) + lo * 2^(sl-127), hi and lo e4m3, sh putting
// the block max in [128, 256) and sl = sh - 4 (clamped at 0).
struct QOperands {
  i32x8_t hi[kSteps];
  i32x8_t lo[kSteps];
  u32x2_t sc_hi, sc_lo;   // byte m (m < 4: .x, else .y) = the lane's scale of step m
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

// The lane's q values of step m as loaded: half h (0, 1) holds the 16
// padded elements 16(grp & 1) .. of block 4m + 2h + grp/2: the block's
// first 16 dims for even lane groups, its last 8 dims and 8 zeros for odd
// ones.
struct QChunk {
  u32x4_t w[4];
};

__device__ __forceinline__ QChunk load_q_chunk(const uint16_t* qh, int m, int grp) {
  QChunk c;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint16_t* bp = qh + kBlk * (4 * m + 2 * h + (grp >> 1));
    if ((grp & 1) == 0) {
      c.w[2 * h] = *(const u32x4_t*)bp;
      c.w[2 * h + 1] = *(const u32x4_t*)(bp + 8);
    } else {
      c.w[2 * h] = *(const u32x4_t*)(bp + 16);
      c.w[2 * h + 1] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  return c;
}

// Split of one step: the e4m3 hi and lo operands and the lane's E8M0 bytes.
// `sign` (0 or 0x80008000) is xored into every pair of bf16 values: a
// negative softmax scale is applied as |scale| on -q, which is exact.
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

// Staging of one split step in LDS (inline-assembly writes: the compiler
// would otherwise hold them behind the tile loads in flight). The writes are
// waited for before the barrier that precedes fetch_q.
__device__ __forceinline__ void stage_q(uint8_t* stage, int m, int lane, const i32x8_t& hi, const i32x8_t& lo,
                                        uint32_t sc_hi, uint32_t sc_lo) {
  const uint32_t a = lds_addr(stage + (m * 2 * 64 + lane) * 32);
  const u32x4_t h0 = {(uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)hi[2], (uint32_t)hi[3]};
  const u32x4_t h1 = {(uint32_t)hi[4], (uint32_t)hi[5], (uint32_t)hi[6], (uint32_t)hi[7]};
  const u32x4_t l0 = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3]};
  const u32x4_t l1 = {(uint32_t)lo[4], (uint32_t)lo[5], (uint32_t)lo[6], (uint32_t)lo[7]};
  asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:16\n\t"
               "ds_write_b128 %0, %3 offset:2048\n\tds_write_b128 %0, %4 offset:2064"
               ::"v"(a), "v"(h0), "v"(h1), "v"(l0), "v"(l1) : "memory");
  const uint32_t sa = lds_addr(stage + kQStage + 8 * lane + m);
  asm volatile("ds_write_b8 %0, %1\n\tds_write_b8 %0, %2 offset:512" ::"v"(sa), "v"(sc_hi), "v"(sc_lo)
               : "memory");
}

template <int M>
__device__ __forceinline__ void fetch_step(uint32_t a, u32x4_t (&r)[4 * kSteps]) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * M + 0]) : "v"(a), "i"(M * 4096));
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * M + 1]) : "v"(a), "i"(M * 4096 + 16));
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * M + 2]) : "v"(a), "i"(M * 4096 + 2048));
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[4 * M + 3]) : "v"(a), "i"(M * 4096 + 2064));
}

__device__ __forceinline__ QOperands fetch_q(const uint8_t* stage, int lane) {
  QOperands f;
  u32x4_t r[4 * kSteps];
  const uint32_t a = lds_addr(stage + lane * 32);
  fetch_step<0>(a, r);
  fetch_step<1>(a, r);
  fetch_step<2>(a, r);
  fetch_step<3>(a, r);
  fetch_step<4>(a, r);
  fetch_step<5>(a, r);
  u32x2_t sh, sl;
  const uint32_t sa = lds_addr(stage + kQStage + 8 * lane);
  asm volatile("ds_read_b64 %0, %1" : "=v"(sh) : "v"(sa));
  asm volatile("ds_read_b64 %0, %1 offset:512" : "=v"(sl) : "v"(sa));
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]),
                 "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]), "+v"(r[12]), "+v"(r[13]), "+v"(r[14]),
                 "+v"(r[15]), "+v"(r[16]), "+v"(r[17]), "+v"(r[18]), "+v"(r[19]), "+v"(r[20]), "+v"(r[21]),
                 "+v"(r[22]), "+v"(r[23]), "+v"(sh), "+v"(sl));
#pragma unroll
  for (int m = 0; m < kSteps; ++m) {
    f.hi[m] = i32x8_t{(int)r[4 * m][0], (int)r[4 * m][1], (int)r[4 * m][2], (int)r[4 * m][3],
                      (int)r[4 * m + 1][0], (int)r[4 * m + 1][1], (int)r[4 * m + 1][2], (int)r[4 * m + 1][3]};
    f.lo[m] = i32x8_t{(int)r[4 * m + 2][0], (int)r[4 * m + 2][1], (int)r[4 * m + 2][2], (int)r[4 * m + 2][3],
                      (int)r[4 * m + 3][0], (int)r[4 * m + 3][1], (int)r[4 * m + 3][2], (int)r[4 * m + 3][3]};
  }
  f.sc_hi = sh;
  f.sc_lo = sl;
  return f;
}

// One MX step of S^T: A = the lane's padded block (three dwords of 24 fp4
// values, then zeros) with its E8M0 byte, B = the step's e4m3 q part with
// scale byte M of `q_scales`.
template <int M>
__device__ __forceinline__ f32x4_t mx_step(const uint32_t (&k)[3], uint32_t k_scale, const i32x8_t& q,
                                           uint32_t q_scales, f32x4_t acc) {
  const i32x8_t a = {(int32_t)k[0], (int32_t)k[1], (int32_t)k[2], 0, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q, acc, 4, 0, 0, (int32_t)k_scale, M,
                                                          (int32_t)q_scales);
}

// S^T = K Q^T for one 16-token sub-tile: returns, for head `col`, the raw
// scores of tokens 16*sub + 4*grp + r (r = 0..3).
__device__ __forceinline__ f32x4_t qk_subtile(const uint8_t* buf, int delta, int sub, const QOperands& qo,
                                              int lane) {
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int row = 16 * sub + col;
  const uint8_t* rp = buf + row * kRowBytes;
  const uint8_t* er = buf + kLdsRaw + delta + kSc * row;
  uint32_t k[kSteps][3];
  uint32_t e[kSteps];
#pragma unroll
  for (int m = 0; m < kSteps; ++m) {
    const uint32_t* kp = (const uint32_t*)(rp + (kBlk / 2) * (4 * m + grp));
    k[m][0] = kp[0];
    k[m][1] = kp[1];
    k[m][2] = kp[2];
    e[m] = er[4 * m + grp];
  }
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  a0 = mx_step<0>(k[0], e[0], qo.hi[0], qo.sc_hi[0], a0);
  a1 = mx_step<0>(k[0], e[0], qo.lo[0], qo.sc_lo[0], a1);
  a0 = mx_step<1>(k[1], e[1], qo.hi[1], qo.sc_hi[0], a0);
  a1 = mx_step<1>(k[1], e[1], qo.lo[1], qo.sc_lo[0], a1);
  a0 = mx_step<2>(k[2], e[2], qo.hi[2], qo.sc_hi[0], a0);
  a1 = mx_step<2>(k[2], e[2], qo.lo[2], qo.sc_lo[0], a1);
  a0 = mx_step<3>(k[3], e[3], qo.hi[3], qo.sc_hi[0], a0);
  a1 = mx_step<3>(k[3], e[3], qo.lo[3], qo.sc_lo[0], a1);
  a0 = mx_step<0>(k[4], e[4], qo.hi[4], qo.sc_hi[1], a0);
  a1 = mx_step<0>(k[4], e[4], qo.lo[4], qo.sc_lo[1], a1);
  a0 = mx_step<1>(k[5], e[5], qo.hi[5], qo.sc_hi[1], a0);
  a1 = mx_step<1>(k[5], e[5], qo.lo[5], qo.sc_lo[1], a1);
  return a0 + a1;
}

// Online-softmax update with the scores of one 32-token tile (s0: tokens
// 4*grp + r of the first sub-tile, s1: of the second, for head `col`):
// returns the tile's hand-off to the P V wave and folds the bf16-rounded P
// into l. `csc` >= 0 (a negative scale reaches here as |scale| with q
// negated); `nvalid` = tokens of the tile inside the item.
__device__ __forceinline__ TileHandoff softmax_tile(f32x4_t s0, f32x4_t s1, int nvalid, SoftmaxState& st,
                                                    float csc, int lane) {
  const int grp = lane >> 4;
  float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  const bool tail = nvalid < kTile;
  if (tail) {   // tokens past the item take no part in the max
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
    // p = 0 past the item, set after the exponential (a zero scale would
    // turn the masked -inf into NaN)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * grp + r >= nvalid) p[r] = 0.f;
      if (16 + 4 * grp + r >= nvalid) p[4 + r] = 0.f;
    }
  }
  const bf16x8_t pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                       (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
  const bf16x8_t ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                         (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  st.l = mfma(pa, ones, st.l);
  h.p = __builtin_bit_cast(u32x4_t, pa);
  return h;
}

// Offset of output block B's first scale block in the formatted table: the
// lanes of B start in scale block floor(4B/3) and move to the next one at
// col 12, 8 or 4 (B mod 3 = 0, 1, 2), which the lane's three addresses hold.
template <int B>
constexpr int fmt_off() { return (4 * B / 3) * (kTile * 4); }

// One output block (32 latent dims) of O += P V: decode the 8 tokens' V bytes
// with their scales and multiply. The reads of block LB + 1 are issued
// before this block's wait so that they overlap its decode.
template <int LB>
__device__ __forceinline__ void pv_block(uint32_t tra, const uint32_t (&sca)[3], u32x2_t& v_cur, u32x4_t& s_lo,
                                         u32x4_t& s_hi, const bf16x8_t& pa, f32x4_t (&o)[32]) {
  u32x2_t v_nx;
  u32x4_t s_nlo, s_nhi;
  if constexpr (LB + 1 < kVBlocks) {
    v_nx = lds_tr8<16 * (LB + 1)>(tra);
    s_nlo = lds_b128<fmt_off<LB + 1>()>(sca[(LB + 1) % 3]);
    s_nhi = lds_b128<fmt_off<LB + 1>() + 16>(sca[(LB + 1) % 3]);
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
  const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, h.p);
  // lane (col, grp) supplies row k = col/2 of its group's 8 tokens, bytes
  // 8*(col&1).. of a 16-byte column block; it receives byte (16B + col) of
  // all 8 tokens (dims 32B + 2col, +1), in the order of the formatted scales.
  const int k = col >> 1;
  const int trow = 4 * grp + (k & 3) + 16 * (k >> 2);
  const uint32_t tra = lds_addr(buf + trow * kRowBytes + 8 * (col & 1));
  const uint32_t base = lds_addr(fmt + 32 * grp);
  const uint32_t sca[3] = {base + (col >= 12 ? kTile * 4 : 0), base + (col >= 8 ? kTile * 4 : 0),
                           base + (col >= 4 ? kTile * 4 : 0)};
  u32x2_t v_cur = lds_tr8<0>(tra);
  u32x4_t s_lo = lds_b128<fmt_off<0>()>(sca[0]), s_hi = lds_b128<fmt_off<0>() + 16>(sca[0]);
  pv_block<0>(tra, sca, v_cur, s_lo, s_hi, pa, o);
}

// One plan item: sequence, token range, partial index (-1: direct output).
struct __attribute__((aligned(16))) ItemWords {
  int32_t b, kb, ke, dest;
};
typedef const __attribute__((address_space(4))) int32_t ConstI32;

__global__ void __launch_bounds__(kThreads, 1)
mla_decode_mxfp4_24_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                           const uint8_t* __restrict__ sc, const int32_t* __restrict__ kv_indptr,
                           uint16_t* __restrict__ out, const int32_t* __restrict__ plan,
                           float* __restrict__ part_lse, float* __restrict__ part_out, float csc) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTotal];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool scorer = (wave >> 2) != 0;   // else the pair's P V wave
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // header words and the first slot's bounds (slot_indptr follows the header
  // in both planners' layouts) in one batch, before the check
  const int32_t* slot_indptr = plan + MLA_PLAN_HEADER_WORDS;
  const int magic = plan[kPwMagic];
  const int version = plan[kPwVersion];
  const int num_slots = plan[kPwNumSlots];
  const int off_items = plan[kPwOffItems];
  int i_begin = slot_indptr[blockIdx.x];
  int i_end = slot_indptr[blockIdx.x + 1];
  // the first slot's first item, from where it sits when the items follow
  // slot_indptr of a launch-sized plan with one item per slot before it;
  // used only if the header and slot_indptr confirm that (the words read
  // are inside the plan whatever it holds: it has at least the launched
  // number of slots, items from this offset on, and an item per slot)
  const int spec_off = (MLA_PLAN_HEADER_WORDS + (int)gridDim.x + 1 + 3) & ~3;
  const ItemWords spec = *(const ItemWords*)(plan + spec_off + 4 * (int)blockIdx.x);
  asm volatile("" ::"s"(num_slots), "s"(off_items), "s"(i_begin), "s"(i_end), "s"(spec.b), "s"(spec.kb),
               "s"(spec.ke), "s"(spec.dest), "s"(q), "s"(kv), "s"(sc), "s"(kv_indptr), "s"(out));
  // only words written by a planner are followed
  if (magic != MLA_PLAN_MAGIC || version != MLA_PLAN_VERSION) return;
  const uint32_t qsign = csc < 0.f ? 0x80008000u : 0u;
  csc = fabsf(csc);

  const int32_t* items = plan + off_items;
  // kv_indptr is not written while the kernel runs: scalar loads through
  // the constant address space
  const ConstI32* kv_indptr_s = (const ConstI32*)kv_indptr;
  uint8_t* ring = lds + pair * kLdsPair;
  TileHandoff* hand = (TileHandoff*)(lds + kLdsXchg) + pair * 64 + lane;  // + parity * kPairs * 64
  uint8_t* fmt_pair = lds + kLdsFmt + pair * kFmtTile;                     // + parity * kPairs * kFmtTile
  uint8_t* qstage = lds + kLdsFmt;
  if (scorer) __builtin_amdgcn_s_setprio(1);

  for (int slot = blockIdx.x; slot < num_slots; slot += gridDim.x) {
    if (slot != (int)blockIdx.x) {
      i_begin = slot_indptr[slot];
      i_end = slot_indptr[slot + 1];
    }
    for (int it = i_begin; it < i_end; ++it) {
      const ItemWords iw = slot == (int)blockIdx.x && it == (int)blockIdx.x && off_items == spec_off
                               ? spec : *(const ItemWords*)(items + 4 * it);
      const int b = iw.b;
      const int dest = iw.dest;
      // the item's rows clamped to the sequence; each role takes them on its
      // own path, the scorer after it has requested q, so that q flies while
      // these scalar loads are waited for
      struct Range {
        int ke, rounds, ntiles, t_first;
      };
      auto item_range = [&]() {
        Range r;
        const int kb = max(iw.kb, kv_indptr_s[b]);
        r.ke = min(iw.ke, kv_indptr_s[b + 1]);
        const int len = r.ke - kb;
        r.rounds = len > 0 ? (len - 1) / kTileStride + 1 : 0;
        const int rel_first = kTile * pair;
        r.ntiles = rel_first < len ? (len - rel_first - 1) / kTileStride + 1 : 0;
        r.t_first = r.ntiles > 0 ? kb + rel_first : kb;
        return r;
      };

      f32x4_t* frag = (f32x4_t*)lds;
      float* stats = (float*)(lds + kMergeFrag);
      if (scorer) {
        SoftmaxState st;
        st.l = f32x4_t{0.f, 0.f, 0.f, 0.f};
        st.m = kMInit;
        // steps pair and (pairs 0, 1) 4 + pair of q, split by this wave
        const uint16_t* qh = q + ((size_t)b * kHeads + col) * kQkDim;
        const QChunk qa = load_q_chunk(qh, pair, grp);
        QChunk qb;
        if (pair < kSteps - 4) qb = load_q_chunk(qh, 4 + pair, grp);
        const Range rg = item_range();
        const int ke = rg.ke, rounds = rg.rounds, ntiles = rg.ntiles, t_first = rg.t_first;
        __syncthreads();  // LDS of the previous item's merge is free again
        // q has landed by now; taking it before tile 0 is requested lets the
        // split run while the tile flies (a wait for q after the tile's
        // loads would also wait for the tile)
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        if (ntiles > 0) stage_dma(ring, kv, sc, t_first, ke - t_first, lane);
        {
          i32x8_t qhi, qlo;
          uint32_t qsh, qsl;
          split_chunk(qa, grp, qsign, qhi, qlo, qsh, qsl);
          stage_q(qstage, pair, lane, qhi, qlo, qsh, qsl);
          if (pair < kSteps - 4) {
            split_chunk(qb, grp, qsign, qhi, qlo, qsh, qsl);
            stage_q(qstage, 4 + pair, lane, qhi, qlo, qsh, qsl);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();  // all six steps staged
        const QOperands qo = fetch_q(qstage, lane);
        for (int i = 0; i <= rounds; ++i) {
          const bool qk_on = i < ntiles;
          if (qk_on) wait_dma();
          __syncthreads();  // tile i landed; tile i-2 fully consumed; hand-off of i-1 visible
          if (i + 1 < ntiles) {
            const int tn = t_first + (i + 1) * kTileStride;
            stage_dma(ring + ((i + 1) % kNumBuf) * kLdsBuf, kv, sc, tn, ke - tn, lane);
          }
          if (qk_on) {
            const int tq = t_first + i * kTileStride;
            const uint8_t* bq = ring + (i % kNumBuf) * kLdsBuf;
            const int dq = raw_delta(sc, tq);
            const f32x4_t s0 = qk_subtile(bq, dq, 0, qo, lane);
            const f32x4_t s1 = qk_subtile(bq, dq, 1, qo, lane);
            hand[(i & 1) * (kPairs * 64)] = softmax_tile(s0, s1, ke - tq, st, csc, lane);
            uint8_t* fm = fmt_pair + (i & 1) * (kPairs * kFmtTile);
            format_scales(bq, fm, dq, ke - tq, lane);
            format_scales(bq, fm, dq, ke - tq, 64 + lane);
            if (lane < kVScaleBlocks * 8 - 128) format_scales(bq, fm, dq, ke - tq, 128 + lane);
          }
        }
        __syncthreads();  // all rounds done: the ring area is free for the merge
        // (the slot index is formed here: an address kept from the prologue
        // would hold a register through the whole item loop)
        int scol = col;
        asm volatile("" : "+v"(scol));
        if (grp == 0) stats[(2 * pair) * kHeads + scol] = st.m;
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
            pv_tile(ring + ((i - 1) % kNumBuf) * kLdsBuf, fmt_pair + ((i - 1) & 1) * (kPairs * kFmtTile), h, o,
                    lane);
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
      // wave w writes output blocks 2w, 2w+1 (both dim parities)
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

}  // namespace

size_t decode_24_lds_bytes() { return (size_t)kLdsTotal; }

int launch_decode_24(const DecodeArgs& a, void* stream) {
  if (a.num_slots <= 0 || a.grid <= 0) return (int)hipSuccess;
  hipLaunchKernelGGL(mla_decode_mxfp4_24_kernel, dim3(a.grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint16_t*)a.q, a.kv_packed, a.kv_scale, a.kv_indptr, (uint16_t*)a.out, a.plan,
                     a.part_lse, a.part_out, a.score_scale_log2);
  return (int)hipGetLastError();
}

}  // namespace mla
