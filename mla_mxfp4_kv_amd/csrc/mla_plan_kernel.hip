// GPU-side planner: the work list of the split-K decode built from a device
// copy of kv_indptr, so that planning needs no host round trip and a caller
// can record plan + decode in one HIP graph while the sequence lengths
// change between replays.
//
// It applies the same slot rule as the host planner (mla_plan.cpp; the pages
// build the work list on the host, page "kernelbot-amd-mixed-mla-608791",
// host metadata builder, and page "kernelbot-amd-mixed-mla-717900" records
// both decode stages in a graph). The host walks slots in order; here each
// sequence is one thread of a single workgroup:
//  * a block scan of the short-sequence flags gives each sequence its start
//    on the weighted line (token offset plus one charge per short sequence
//    before it) and so the start tok0 of its tokens there;
//  * a non-empty sequence of n tokens overlaps slots s0 = tok0 / chunk ..
//    s1 = (tok0 + n - 1) / chunk and has one item per slot;
//  * sequences and slots are both contiguous and ascending, so ordering the
//    items by slot and then by sequence is the same as ordering them by
//    sequence and then by slot: a sequence's first item index is the
//    exclusive prefix sum of the pieces of the sequences before it;
//  * partial indices number the pieces of split sequences (two or more
//    pieces) in the same order, reduce entries the split or empty sequences;
//  * a sequence writes slot_indptr[s] for every slot it enters first: slots
//    s0 < s <= s1, and s0 itself when no earlier sequence has tokens in it
//    (the earlier tokens end at or before the slot's start).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

struct Counts {
  int32_t items, partials, reduce;
};

// Exclusive prefix sums of the three counts over the workgroup's threads, in
// thread order; `total` receives the workgroup sums. All threads call it.
__device__ Counts block_exclusive_scan(Counts v, Counts* total, Counts* s_wave) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  Counts inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t a = __shfl_up(inc.items, d), b = __shfl_up(inc.partials, d), c = __shfl_up(inc.reduce, d);
    if (lane >= d) {
      inc.items += a;
      inc.partials += b;
      inc.reduce += c;
    }
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  Counts before = {0, 0, 0}, all = {0, 0, 0};
  for (int w = 0; w < kPlanWaves; ++w) {
    const Counts t = s_wave[w];
    if (w < wave) {
      before.items += t.items;
      before.partials += t.partials;
      before.reduce += t.reduce;
    }
    all.items += t.items;
    all.partials += t.partials;
    all.reduce += t.reduce;
  }
  __syncthreads();   // s_wave may be reused by the next call
  *total = all;
  return Counts{before.items + inc.items - v.items, before.partials + inc.partials - v.partials,
                before.reduce + inc.reduce - v.reduce};
}

__global__ void __launch_bounds__(kPlanThreads)
mla_plan_kernel(const int32_t* __restrict__ ind, int32_t batch, int32_t num_cus, int64_t max_total,
                int32_t off_items, int32_t off_reduce, int32_t off_lse, int32_t off_out,
                int32_t* __restrict__ w) {
  __shared__ Counts s_wave[kPlanWaves];
  const int tid = threadIdx.x;
  const int64_t base = ind[0];
  const int64_t end = ind[batch];
  const int64_t total = end - base;
  int bad = base < 0 || total < 0 || total > max_total || end > INT32_MAX;
  for (int b = tid; b < batch; b += kPlanThreads) bad |= ind[b + 1] < ind[b];
  bad = __syncthreads_or(bad);

  const int64_t g = (int64_t)num_cus * MLA_PLAN_WG_PER_CU;
  // Item charges (the host planner's rule): when the equal-token slot c0 is
  // longer than an item's fixed work, a sequence shorter than c0 takes
  // MLA_PLAN_ITEM_COST units ahead of its tokens on the weighted line.
  int64_t c0 = 0;
  if (!bad && total > 0) {
    const int64_t per = (total + g - 1) / g;
    const int64_t aligned = (per + MLA_PLAN_CHUNK_ALIGN - 1) / MLA_PLAN_CHUNK_ALIGN * MLA_PLAN_CHUNK_ALIGN;
    c0 = aligned > MLA_PLAN_MIN_CHUNK ? aligned : MLA_PLAN_MIN_CHUNK;
  }
  const bool charge = c0 > MLA_PLAN_ITEM_COST;
  auto is_short = [&](int b) {
    const int64_t len = (int64_t)ind[b + 1] - ind[b];
    return charge && len > 0 && len < c0;
  };
  int64_t num_short = 0;
  for (int b0 = 0; charge && b0 < batch; b0 += kPlanThreads)
    num_short += __syncthreads_count(b0 + tid < batch && is_short(b0 + tid));
  const int64_t wt = total + (int64_t)MLA_PLAN_ITEM_COST * num_short;

  int64_t chunk = 0, num_slots = 0;
  if (!bad && total > 0) {
    const int64_t per = (wt + g - 1) / g;
    const int64_t aligned = (per + MLA_PLAN_CHUNK_ALIGN - 1) / MLA_PLAN_CHUNK_ALIGN * MLA_PLAN_CHUNK_ALIGN;
    chunk = aligned > MLA_PLAN_MIN_CHUNK ? aligned : MLA_PLAN_MIN_CHUNK;
    num_slots = (wt + chunk - 1) / chunk;
  }
  int32_t* slot_indptr = w + MLA_PLAN_HEADER_WORDS;
  int32_t* items = w + off_items;
  int32_t* red = w + off_reduce;

  Counts carry = {0, 0, 0};
  int64_t short_carry = 0;
  for (int b0 = 0; !bad && b0 < batch; b0 += kPlanThreads) {
    const int b = b0 + tid;
    // where this sequence starts on the weighted line: its tokens' offset
    // plus one charge per short sequence before it
    const int sh_b = b < batch && is_short(b) ? 1 : 0;
    Counts short_sum;
    const int64_t shorts_before =
        short_carry + block_exclusive_scan(Counts{sh_b, 0, 0}, &short_sum, s_wave).items;
    short_carry += short_sum.items;

    int64_t sl = 0, sh = 0, s0 = 0, tok0 = 0, line_start = 0;
    Counts mine = {0, 0, 0};
    if (b < batch) {
      sl = ind[b];
      sh = ind[b + 1];
      line_start = (sl - base) + (int64_t)MLA_PLAN_ITEM_COST * shorts_before;
      tok0 = line_start + (int64_t)MLA_PLAN_ITEM_COST * sh_b;
      if (sh > sl) {
        s0 = tok0 / chunk;
        const int64_t s1 = (tok0 + (sh - sl) - 1) / chunk;
        mine.items = (int32_t)(s1 - s0 + 1);
        mine.partials = mine.items >= 2 ? mine.items : 0;
        mine.reduce = mine.items >= 2;
      } else {
        mine.reduce = 1;   // empty: the reduce writes zeros
      }
    }
    Counts sum;
    const Counts ex = block_exclusive_scan(mine, &sum, s_wave);
    if (b < batch) {
      const int32_t first_item = carry.items + ex.items;
      const int32_t first_partial = carry.partials + ex.partials;
      const int64_t tok1 = tok0 + (sh - sl);
      for (int k = 0; k < mine.items; ++k) {
        const int64_t s = s0 + k;
        const int64_t lo = s * chunk, hi = lo + chunk;
        const int64_t u0 = lo > tok0 ? lo : tok0, u1 = hi < tok1 ? hi : tok1;
        int32_t* it = items + 4 * (first_item + k);
        it[0] = b;
        it[1] = (int32_t)(sl + (u0 - tok0));
        it[2] = (int32_t)(sl + (u1 - tok0));
        it[3] = mine.partials ? first_partial + k : -1;
        // first item of slot s: the slot starts inside this sequence's
        // tokens, or the tokens before it end at or before the slot start
        if (k > 0 || line_start <= lo) slot_indptr[s] = first_item + k;
      }
      if (mine.reduce) {
        int32_t* r = red + 4 * (carry.reduce + ex.reduce);
        r[0] = b;
        r[1] = mine.partials ? first_partial : 0;
        r[2] = mine.items;
        r[3] = 0;
      }
    }
    carry.items += sum.items;
    carry.partials += sum.partials;
    carry.reduce += sum.reduce;
  }

  if (tid == 0) {
    if (!bad) slot_indptr[num_slots] = carry.items;
    // An invalid indptr leaves an empty plan (no slots, no reduce entries)
    // with magic 0: the decode then enqueues kernels that do nothing.
    w[kPwMagic] = bad ? 0 : MLA_PLAN_MAGIC;
    w[kPwVersion] = MLA_PLAN_VERSION;
    w[kPwBatch] = batch;
    w[kPwBase] = (int32_t)base;
    w[kPwTotal] = bad ? 0 : (int32_t)total;
    w[kPwNumCus] = num_cus;
    w[kPwChunk] = (int32_t)(chunk < INT32_MAX ? chunk : INT32_MAX);   // a record of the rule's value
    w[kPwNumSlots] = (int32_t)num_slots;
    w[kPwNumItems] = carry.items;
    w[kPwNumPartials] = carry.partials;
    w[kPwNumReduce] = carry.reduce;
    w[kPwOffSlot] = MLA_PLAN_HEADER_WORDS;
    w[kPwOffItems] = off_items;
    w[kPwOffReduce] = off_reduce;
    w[kPwOffLse] = off_lse;
    w[kPwOffOut] = off_out;
  }
}

}  // namespace

int launch_plan_device(const int32_t* kv_indptr, int32_t batch, int32_t num_cus, int64_t max_total,
                       const DeviceLayout& l, void* workspace, void* stream) {
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream, kv_indptr,
                     batch, num_cus, max_total, (int32_t)l.off_items, (int32_t)l.off_reduce,
                     (int32_t)l.off_lse, (int32_t)l.off_out, (int32_t*)workspace);
  return (int)hipGetLastError();
}

}  // namespace mla
