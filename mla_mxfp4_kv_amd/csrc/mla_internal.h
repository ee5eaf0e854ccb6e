// Internal declarations shared by the host API, the planner and the kernels
// of libmla_mxfp4.so. Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "mla_mxfp4.h"

namespace mla {

// Plan header word indices (int32 words at the start of the workspace).
enum PlanWord : int {
  kPwMagic = 0,
  kPwVersion = 1,
  kPwBatch = 2,
  kPwBase = 3,
  kPwTotal = 4,
  kPwNumCus = 5,
  kPwChunk = 6,
  kPwNumSlots = 7,
  kPwNumItems = 8,
  kPwNumPartials = 9,
  kPwNumReduce = 10,
  kPwOffSlot = 11,      // word offset of slot_indptr[num_slots + 1]
  kPwOffItems = 12,     // word offset of items[num_items][4] = {b, kv_begin, kv_end, dest}
  kPwOffReduce = 13,    // word offset of reduce[num_reduce][4] = {b, first, count, 0}
  kPwOffLse = 14,       // byte offset of partial LSE   float [P][16]
  kPwOffOut = 15,       // byte offset of partial output float [P][16][512]
};

constexpr int kAlignBytes = 256;

struct PlanResult {
  std::vector<int32_t> words;
  size_t workspace_bytes = 0;
  int32_t num_slots = 0;
  int32_t num_reduce = 0;
  int32_t num_partials = 0;
  int32_t off_lse = 0;
  int32_t off_out = 0;
};

// Host planner (mla_plan.cpp). Returns MLA_OK or MLA_ERR_INVALID with *err set.
int build_plan(const int32_t* kv_indptr, int32_t batch, int32_t num_cus,
               PlanResult* out, std::string* err);

// Upper bound on the workspace for any indptr of this size (mla_plan.cpp).
size_t workspace_bound(int32_t batch, int64_t total, int32_t num_cus);

// Plan layout sized for the bounds (batch sequences, at most max_total
// tokens) rather than for one indptr: what the GPU-side planner fills
// (mla_plan.cpp). Its total_bytes equals workspace_bound().
struct DeviceLayout {
  int64_t slots;        // bound on the slot count
  int64_t off_items, off_reduce, off_lse, off_out, total_bytes;
};
DeviceLayout device_layout(int32_t batch, int64_t max_total, int32_t num_cus);

// Kernel launchers (mla_kernels.hip). Return the hipError_t of the launch as int.
struct DecodeArgs {
  const void* q;
  const uint8_t* kv_packed;
  const uint8_t* kv_scale;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;   // per-token cache rows, or pages (nullptr: contiguous sequences)
  const int32_t* page_indptr;  // with pages: sequence b's pages start at kv_indices[page_indptr[b]]
                               // (nullptr: kv_indices lists one row per token)
  int32_t page_size;           // rows per page (1 for a per-token row list)
  const int32_t* kv_start;     // contiguous rows: sequence b starts at row kv_start[b]
                               // (nullptr: at kv_indptr[b])
  void* out;
  const int32_t* plan;    // device plan words (workspace start)
  float* part_lse;
  float* part_out;
  float score_scale_log2;  // sm_scale * log2(e)
  int32_t num_slots;
  int32_t num_reduce;
  int32_t grid;            // decode workgroups to launch
  int32_t wide_reduce;     // 1: merge with 16 waves per (sequence, head, dim quarter)
                           // (long splits); 0: one wave per (sequence, head)
};

// GPU-side planner launch (mla_plan_kernel.hip).
int launch_plan_device(const int32_t* kv_indptr, int32_t batch, int32_t num_cus, int64_t max_total,
                       const DeviceLayout& l, void* workspace, void* stream);

int launch_decode(const DecodeArgs& a, void* stream);
int launch_reduce(const DecodeArgs& a, void* stream);

// fp8 / bf16 cache decode (mla_dense_kernels.hip): the same plan, partials
// and reduce; a.kv_packed holds the cache rows, kv_scale the device pointer
// of the fp8 per-tensor scale (unused for bf16).
int launch_decode_dense(const DecodeArgs& a, bool fp8, const float* kv_scale, void* stream);

// Static device scratch of mla_decode_mxfp4_noalloc (mla_noalloc.hip): its
// size, and the device address of the current device's copy (looked up
// once per device; returns the hipError_t as int).
constexpr size_t kNoAllocScratchBytes = (size_t)20 << 20;
int noalloc_scratch(int device, void** ptr);

// 24-scale MXFP4 decode (mla_mxfp4_24_kernels.hip): a.kv_scale holds the
// [T, 24] E8M0 rows (8-byte aligned); contiguous rows only.
int launch_decode_24(const DecodeArgs& a, void* stream);

// Static LDS bytes the decode kernels need (for validation against the device).
size_t decode_lds_bytes();
size_t decode_dense_lds_bytes();
size_t decode_24_lds_bytes();

}  // namespace mla
