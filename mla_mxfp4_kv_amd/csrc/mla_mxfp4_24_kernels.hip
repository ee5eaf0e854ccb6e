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
// The 24-element blocks do not match the 32-element scale blocks of the
// MX-scaled MFMA, so both products run on the bf16 MFMA with K and V decoded
// in registers by the scaled fp4 converter (exact for scale bytes whose
// products stay normal in bf16). Structure (one workgroup of 4 waves per CU,
// one wave per SIMD, persistent over the planner's slots):
//  * a wave takes every 4th 32-token tile of its item; the tile's packed rows
//    (9 KB, as in memory) and its scale rows (768 bytes, as the 16-byte
//    chunks covering them) go straight to the wave's own LDS ring of three
//    buffers, two tiles ahead of the one computed;
//  * QK (S^T = K Q^T, 16 heads as the MFMA N dimension): lane group g takes
//    the 144 contiguous dims 144g .. 144g+143 -- six whole scale blocks --
//    so each 8-dim K step of a lane has one scale and the lane reads its
//    72 packed bytes contiguously; q is loaded in the same dim order;
//  * online softmax in base 2 (scale first, then the tail mask, then the max,
//    lazily raised by more than 8), P rounded to bf16, l summed from it;
//  * P V: V bytes read transposed (ds_read_b64_tr_b8: a lane receives byte
//    column 16B + col of its 8 tokens = dims 32B + 2col, +1), decoded token
//    by token with the scale of block (32B + 2col) / 24, which the tile's
//    formatted scale table gives per (block, token); the even and odd dims
//    of a 32-dim block are two MFMA output tiles;
//  * the 4 waves' (m, l, O) merge through LDS; whole sequences write bf16,
//    split items a normalised fp32 partial and its base-2 LSE.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#define MLA_LDS __attribute__((address_space(3)))

constexpr int kHeads = MLA_NUM_HEADS;
constexpr int kQkDim = MLA_QK_DIM;
constexpr int kVDim = MLA_V_DIM;
constexpr int kRow = MLA_PACKED_BYTES;          // 288
constexpr int kSc = MLA_SCALES_PER_TOKEN_24;    // 24
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                       // tokens per wave tile
constexpr int kStride = kWaves * kTile;         // a wave's step through the item
constexpr int kRowDma = kTile * kRow / 1024;    // 9 instructions of 1 KB
constexpr int kRaw = kTile * kRow;              // the tile's scale chunks after its rows
constexpr int kRawChunks = (kTile * kSc) / 16 + 1;   // 49 chunks cover 768 bytes at an 8-byte offset
constexpr int kBuf = kRaw + kRawChunks * 16 + 48;    // 10048 (multiple of 64)
constexpr int kNumBuf = 3;
constexpr int kVBlocks24 = (kVDim + 23) / 24;   // 22 scale blocks hold a V dim
constexpr int kFmt = kVBlocks24 * kTile * 4;    // formatted V scales: [block][position] dwords
constexpr int kWaveLds = kNumBuf * kBuf + kFmt;
constexpr int kOFrags = kVDim / 16;             // 32 output tiles of 16 dims
constexpr int kMergeFrag = kWaves * kOFrags * 64 * 16;
constexpr int kMergeBytes = kMergeFrag + kWaves * 2 * kHeads * 4;
constexpr int kLdsRing = kWaves * kWaveLds;
constexpr int kLdsTotal = kLdsRing > kMergeBytes ? kLdsRing : kMergeBytes;
constexpr float kTau = 8.0f;
constexpr int kStream = 2;                      // non-temporal tile loads
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1.0e30f;

static_assert(kLdsTotal <= 160 * 1024, "LDS budget of one gfx950 CU");
static_assert(kBuf % 64 == 0 && kWaveLds % 16 == 0, "buffers stay aligned");
static_assert(kQkDim == 4 * 144, "four lane groups of 144 dims");

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS uint8_t*)p;
}

// Stage the 32-token tile starting at token t0 (`nvalid` tokens of it inside
// the item) into `buf` with direct global->LDS loads: the packed rows as one
// contiguous copy (rows past the last valid one repeat its last 16 bytes),
// then the 16-byte chunks that cover the tile's scale rows, so that scale
// byte (row, k) lands at buf + kRaw + delta + 24 row + k with delta = the
// first byte's offset in its chunk (0 or 8: scale rows are 8-byte aligned).
__device__ __forceinline__ void stage_tile(uint8_t* buf, const uint8_t* __restrict__ kv,
                                           const uint8_t* __restrict__ sc, int t0, int nvalid, int lane) {
  t0 = __builtin_amdgcn_readfirstlane(t0);
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  const uint8_t* src = kv + (size_t)t0 * kRow;
  const uint32_t lane_off = 16 * lane;
  if (nvalid >= kTile) {
#pragma unroll
    for (int i = 0; i < kRowDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + 1024 * i + lane_off), (MLA_LDS void*)(buf + 1024 * i),
                                       16, 0, kStream);
  } else {
    const uint32_t last = (uint32_t)(nvalid * kRow - 16);
#pragma unroll
    for (int i = 0; i < kRowDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + min(1024 * i + lane_off, last)),
                                       (MLA_LDS void*)(buf + 1024 * i), 16, 0, kStream);
  }
  const uintptr_t first = (uintptr_t)(sc + (size_t)t0 * kSc);
  const uintptr_t last_chunk = (first + (uintptr_t)(kSc * min(nvalid, kTile)) - 1) & ~(uintptr_t)15;
  const uintptr_t csrc = min((first & ~(uintptr_t)15) + lane_off, last_chunk);
  if (lane < kRawChunks)
    __builtin_amdgcn_global_load_lds((const void*)csrc, (MLA_LDS void*)(buf + kRaw), 16, 0, kStream);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float max_over_groups(float v) {
  // max over lanes h, h+16, h+32, h+48; the swap results are copied to
  // scalars before their bit casts (a bit cast of a vector element reads
  // element 0)
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float m1 = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t u1 = __builtin_bit_cast(uint32_t, m1);
  const auto c = __builtin_amdgcn_permlane16_swap(u1, u1, false, false);
  const uint32_t c0 = c[0], c1 = c[1];
  return fmaxf(__builtin_bit_cast(float, c0), __builtin_bit_cast(float, c1));
}

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// 8 e2m1 codes (a dword, low nibble first) times 2^(e-127) -> 8 bf16; the
// scale operand is the exponent-field float of the E8M0 byte.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float s) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// q of head `col` as the B operands of the 18 K steps: step s = 3j + u holds
// dims 144 grp + 24 j + 8 u .. +7 (block 6 grp + j, its u-th 8 dims).
struct Q24 {
  bf16x8_t q[18];
};

__device__ __forceinline__ Q24 load_q24(const uint16_t* qh, int grp) {
  Q24 f;
#pragma unroll
  for (int j = 0; j < 6; ++j)
#pragma unroll
    for (int u = 0; u < 3; ++u) f.q[3 * j + u] = *(const bf16x8_t*)(qh + 144 * grp + 24 * j + 8 * u);
  return f;
}

// Raw scores (before the softmax scale) of tokens 16 sub + 4 grp + r for head
// `col`. Lane (col, grp) supplies K row 16 sub + col: its 72 packed bytes at
// 72 grp (dims 144 grp ..) and the 6 scale bytes 6 grp .. 6 grp + 5.
__device__ __forceinline__ f32x4_t scores24(const uint8_t* buf, int delta, int sub, const Q24& qo, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  const int row = 16 * sub + col;
  const uint32_t ka = lds_addr(buf + row * kRow + 72 * grp);
  u32x2_t k[9];
  const uint32_t sa = lds_addr(buf + kRaw + delta + kSc * row + 6 * grp);
  const uint32_t s4 = sa & ~3u;
  uint32_t sw[3];
  asm volatile(
      "ds_read_b64 %0, %12 offset:0\n\t"
      "ds_read_b64 %1, %12 offset:8\n\t"
      "ds_read_b64 %2, %12 offset:16\n\t"
      "ds_read_b64 %3, %12 offset:24\n\t"
      "ds_read_b64 %4, %12 offset:32\n\t"
      "ds_read_b64 %5, %12 offset:40\n\t"
      "ds_read_b64 %6, %12 offset:48\n\t"
      "ds_read_b64 %7, %12 offset:56\n\t"
      "ds_read_b64 %8, %12 offset:64\n\t"
      "ds_read_b32 %9, %13 offset:0\n\t"
      "ds_read_b32 %10, %13 offset:4\n\t"
      "ds_read_b32 %11, %13 offset:8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]),
        "=&v"(k[8]), "=&v"(sw[0]), "=&v"(sw[1]), "=&v"(sw[2])
      : "v"(ka), "v"(s4));
  // the 6 scale bytes as exponent-field floats
  const uint32_t sh = 8 * (sa & 3u);
  const uint32_t w0 = (uint32_t)(((uint64_t)sw[1] << 32 | sw[0]) >> sh);
  const uint32_t w1 = (uint32_t)(((uint64_t)sw[2] << 32 | sw[1]) >> sh);
  const uint32_t eb[6] = {w0 & 0xFFu, (w0 >> 8) & 0xFFu, (w0 >> 16) & 0xFFu, w0 >> 24, w1 & 0xFFu, (w1 >> 8) & 0xFFu};
  uint32_t kd[18];
#pragma unroll
  for (int d = 0; d < 9; ++d) {
    const u32x2_t kv2 = k[d];
    const uint32_t lo = kv2[0], hi = kv2[1];
    kd[2 * d] = lo;
    kd[2 * d + 1] = hi;
  }
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const float s = __builtin_bit_cast(float, eb[j] << 23);
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int st = 3 * j + u;
      if (st & 1) a1 = mfma(dequant8(kd[st], s), qo.q[st], a1);
      else a0 = mfma(dequant8(kd[st], s), qo.q[st], a0);
    }
  }
  return a0 + a1;
}

// Formatted V scales of a landed tile: F[block][position] = exponent-field
// dword of the token's scale byte for 24-element block `block` (0..21),
// position 8g + j = token 4g + (j & 3) + 16 (j >> 2) (the order in which lane
// group g holds P). Rows at or past `nvalid` get scale 1 (their p is 0, and
// a stale byte must not turn 0 * V into NaN). Lane l < 44 writes block l / 2,
// positions 16 (l & 1) ..
__device__ __forceinline__ void format24(const uint8_t* buf, uint8_t* fmt, int delta, int nvalid, int lane) {
  if (lane < 2 * kVBlocks24) {
    const int blk = lane >> 1;
    const int half = lane & 1;   // positions 16 half .. : lane groups 2 half, 2 half + 1
    // position 16 half + k is token R(k) + 8 half, R(k) = 4 (k >> 3) + (k & 3) + 16 ((k >> 2) & 1)
    const uint32_t ra = lds_addr(buf + kRaw + delta + blk + kSc * 8 * half);
    uint32_t e[16];
    // LDS accesses from inline assembly, waited for inside the block: the
    // compiler would otherwise wait for the tile loads in flight first
    asm volatile(
        "ds_read_u8 %0, %16 offset:%17\n\t"
        "ds_read_u8 %1, %16 offset:%18\n\t"
        "ds_read_u8 %2, %16 offset:%19\n\t"
        "ds_read_u8 %3, %16 offset:%20\n\t"
        "ds_read_u8 %4, %16 offset:%21\n\t"
        "ds_read_u8 %5, %16 offset:%22\n\t"
        "ds_read_u8 %6, %16 offset:%23\n\t"
        "ds_read_u8 %7, %16 offset:%24\n\t"
        "ds_read_u8 %8, %16 offset:%25\n\t"
        "ds_read_u8 %9, %16 offset:%26\n\t"
        "ds_read_u8 %10, %16 offset:%27\n\t"
        "ds_read_u8 %11, %16 offset:%28\n\t"
        "ds_read_u8 %12, %16 offset:%29\n\t"
        "ds_read_u8 %13, %16 offset:%30\n\t"
        "ds_read_u8 %14, %16 offset:%31\n\t"
        "ds_read_u8 %15, %16 offset:%32\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(e[0]), "=&v"(e[1]), "=&v"(e[2]), "=&v"(e[3]), "=&v"(e[4]), "=&v"(e[5]), "=&v"(e[6]), "=&v"(e[7]),
          "=&v"(e[8]), "=&v"(e[9]), "=&v"(e[10]), "=&v"(e[11]), "=&v"(e[12]), "=&v"(e[13]), "=&v"(e[14]),
          "=&v"(e[15])
        : "v"(ra), "i"(kSc * 0), "i"(kSc * 1), "i"(kSc * 2), "i"(kSc * 3), "i"(kSc * 16), "i"(kSc * 17),
          "i"(kSc * 18), "i"(kSc * 19), "i"(kSc * 4), "i"(kSc * 5), "i"(kSc * 6), "i"(kSc * 7), "i"(kSc * 20),
          "i"(kSc * 21), "i"(kSc * 22), "i"(kSc * 23));
    u32x4_t v[4];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = 4 * (k >> 3) + (k & 3) + 16 * ((k >> 2) & 1) + 8 * half;
      v[k >> 2][k & 3] = (row < nvalid ? e[k] : 127u) << 23;
    }
    const uint32_t wa = lds_addr(fmt + blk * (kTile * 4) + 64 * half);
    asm volatile(
        "ds_write_b128 %0, %1 offset:0\n\t"
        "ds_write_b128 %0, %2 offset:16\n\t"
        "ds_write_b128 %0, %3 offset:32\n\t"
        "ds_write_b128 %0, %4 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)" ::"v"(wa), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])
        : "memory");
  }
}

// One 32-dim block DB of O += P V: the lane's byte column decoded token by
// token with the scale of its 24-element block (32 DB + 2 col) / 24 -- one
// of the two blocks the 32 dims touch -- then regrouped into token pairs
// (even dims, odd dims) for two MFMAs with the tile's 32 tokens as K.
template <int DB>
__device__ __forceinline__ void pv_block24(uint32_t tra, uint32_t fmt_lane, int col, const bf16x8_t& pa,
                                           f32x4_t (&o)[kOFrags]) {
  constexpr int kB0 = (32 * DB) / 24;                  // block of dim 32 DB
  constexpr int kThr = 24 * (kB0 + 1) - 32 * DB;       // first in-block offset of the next block
  const uint32_t fa = fmt_lane + (uint32_t)((kB0 + (2 * col >= kThr ? 1 : 0)) * kTile * 4);
  u32x2_t v;
  u32x4_t s_lo, s_hi;
  asm volatile(
      "ds_read_b64_tr_b8 %0, %3 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:0\n\t"
      "ds_read_b128 %2, %4 offset:16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v), "=&v"(s_lo), "=&v"(s_hi)
      : "v"(tra), "v"(fa), "i"(16 * DB));
  const uint32_t sv[8] = {s_lo[0], s_lo[1], s_lo[2], s_lo[3], s_hi[0], s_hi[1], s_hi[2], s_hi[3]};
  const uint32_t v0 = v[0], v1 = v[1];
  uint32_t c[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const float scl = __builtin_bit_cast(float, sv[kk]);
    const uint32_t src = kk < 4 ? v0 : v1;
    bf16x2_t cv;
    switch (kk & 3) {
      case 0: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 0); break;
      case 1: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 1); break;
      case 2: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 2); break;
      default: cv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 3); break;
    }
    c[kk] = __builtin_bit_cast(uint32_t, cv);
  }
  const u32x4_t be = {__builtin_amdgcn_perm(c[1], c[0], 0x05040100u), __builtin_amdgcn_perm(c[3], c[2], 0x05040100u),
                      __builtin_amdgcn_perm(c[5], c[4], 0x05040100u), __builtin_amdgcn_perm(c[7], c[6], 0x05040100u)};
  const u32x4_t bo = {__builtin_amdgcn_perm(c[1], c[0], 0x07060302u), __builtin_amdgcn_perm(c[3], c[2], 0x07060302u),
                      __builtin_amdgcn_perm(c[5], c[4], 0x07060302u), __builtin_amdgcn_perm(c[7], c[6], 0x07060302u)};
  o[2 * DB] = mfma(pa, __builtin_bit_cast(bf16x8_t, be), o[2 * DB]);
  o[2 * DB + 1] = mfma(pa, __builtin_bit_cast(bf16x8_t, bo), o[2 * DB + 1]);
  if constexpr (DB + 1 < kVDim / 32) pv_block24<DB + 1>(tra, fmt_lane, col, pa, o);
}

__global__ void __launch_bounds__(kThreads, 1)
mla_decode_mxfp4_24_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                           const uint8_t* __restrict__ sc, const int32_t* __restrict__ kv_indptr,
                           uint16_t* __restrict__ out, const int32_t* __restrict__ plan,
                           float* __restrict__ part_lse, float* __restrict__ part_out, float csc) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTotal];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // header words in one batch (the compiler would fetch each only after the
  // previous check); only words written by a planner are followed
  const int magic = plan[kPwMagic];
  const int version = plan[kPwVersion];
  const int num_slots = plan[kPwNumSlots];
  const int off_slot = plan[kPwOffSlot];
  const int off_items = plan[kPwOffItems];
  asm volatile("" ::"s"(num_slots), "s"(off_slot), "s"(off_items), "s"(q), "s"(kv), "s"(sc), "s"(kv_indptr),
               "s"(out));
  if (magic != MLA_PLAN_MAGIC || version != MLA_PLAN_VERSION) return;

  const int32_t* slot_indptr = plan + off_slot;
  const int32_t* items = plan + off_items;
  uint8_t* ring = lds + wave * kWaveLds;
  uint8_t* fmt = ring + kNumBuf * kBuf;
  f32x4_t* frag = (f32x4_t*)lds;
  float* stats = (float*)(lds + kMergeFrag);
  // P V lane constants: the row this lane supplies to the transposing read
  // (row k = col / 2 of its group's 8 tokens, half col & 1 of the 16-byte
  // column), and its group's slot in the formatted scale table
  const int kr = col >> 1;
  const int trow = 4 * grp + (kr & 3) + 16 * (kr >> 2);

  for (int slot = blockIdx.x; slot < num_slots; slot += gridDim.x) {
    const int i_begin = slot_indptr[slot];
    const int i_end = slot_indptr[slot + 1];
    for (int it = i_begin; it < i_end; ++it) {
      const int b = items[4 * it + 0];
      const int kb = max(items[4 * it + 1], kv_indptr[b]);
      const int ke = min(items[4 * it + 2], kv_indptr[b + 1]);
      const int dest = items[4 * it + 3];
      // counts from differences: offsets near 2^31 - 1 cannot wrap
      const int len = ke - kb;
      const int rel_first = kTile * wave;
      const int ntiles = rel_first < len ? (len - rel_first - 1) / kStride + 1 : 0;
      const int t_first = ntiles > 0 ? kb + rel_first : kb;

      Q24 qo = load_q24(q + ((size_t)b * kHeads + col) * kQkDim, grp);
      // take the q loads here, so that no wait for them (which would also
      // wait for the tile loads) lands in the tile loop
#pragma unroll
      for (int s = 0; s < 18; ++s) asm volatile("" : "+v"(qo.q[s]));

      float m = kMInit;    // running max of head col (base-2 scaled scores)
      float l = 0.f;       // this lane's share of head col's denominator
      f32x4_t o[kOFrags];
#pragma unroll
      for (int n = 0; n < kOFrags; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      __syncthreads();   // the previous item's merge has read the merge area
      if (ntiles > 0) stage_tile(ring, kv, sc, t_first, ke - t_first, lane);
      if (ntiles > 1) stage_tile(ring + kBuf, kv, sc, t_first + kStride, ke - t_first - kStride, lane);
      for (int i = 0; i < ntiles; ++i) {
        // tile i + 2 goes into the buffer of tile i - 1 before tile i is
        // waited for; each tile is 10 loads and they complete in order
        if (i + 2 < ntiles) {
          const int tn = t_first + (i + 2) * kStride;
          stage_tile(ring + ((i + 2) % kNumBuf) * kBuf, kv, sc, tn, ke - tn, lane);
          wait_vm<2 * (kRowDma + 1)>();
        } else if (i + 1 < ntiles) {
          wait_vm<kRowDma + 1>();
        } else {
          wait_vm<0>();
        }
        const int t0 = t_first + i * kStride;
        const int nvalid = ke - t0;
        const uint8_t* buf = ring + (i % kNumBuf) * kBuf;
        const int delta = (int)((uintptr_t)(sc + (size_t)t0 * kSc) & 15);

        format24(buf, fmt, delta, nvalid, lane);
        const f32x4_t s0 = scores24(buf, delta, 0, qo, lane);
        const f32x4_t s1 = scores24(buf, delta, 1, qo, lane);
        float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= csc;   // scaled first: any sign of the scale
        if (nvalid < kTile) {                      // tail tile: tokens past the item get p = 0
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (4 * grp + r >= nvalid) x[r] = kNegInf;
            if (16 + 4 * grp + r >= nvalid) x[4 + r] = kNegInf;
          }
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
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
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = (float)(__bf16)__builtin_amdgcn_exp2f(x[j] - m);
          l += p[j];
        }
        const bf16x8_t pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                             (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        pv_block24<0>(lds_addr(buf + trow * kRow + 8 * (col & 1)), lds_addr(fmt + 32 * grp), col, pa, o);
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
        inv[r] = lsum != 0.f ? 1.0f / lsum : 0.f;
        lse[r] = lsum != 0.f ? mmax + __builtin_amdgcn_logf(lsum) : kNegInf;
      }
      // wave w writes 32-dim blocks 4w .. 4w + 3 (fragment 2 blk: even dims
      // 32 blk + 2 col, fragment 2 blk + 1: the odd ones)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int blk = 4 * wave + bb;
        f32x4_t ev = {0.f, 0.f, 0.f, 0.f}, od = ev;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const f32x4_t fe = frag[(w * kOFrags + 2 * blk) * 64 + lane];
          const f32x4_t fo = frag[(w * kOFrags + 2 * blk + 1) * 64 + lane];
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
            float* pp = part_out + ((size_t)dest * kHeads + h) * kVDim + d;
            pp[0] = re;
            pp[1] = ro;
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
