// Host work-list planner for the split-K decode.
//
// The pages build the work list on the host: one row per (batch, KV range)
// with the index of the partial it writes, plus a per-batch list of the
// partials to merge (kernelindex page "kernelbot-amd-mixed-mla-608791",
// host metadata builder). They cut every sequence into fixed 128-token
// chunks. Here the concatenated token stream is cut into `num_slots` equal
// contiguous slots, one per workgroup of the device, so every workgroup
// streams the same number of KV bytes whatever the length mix; slots are then
// cut at sequence boundaries into items. When workgroups have more than an
// item's fixed work to stream, short sequences are charged that work, so a
// slot that holds several of them gets fewer tokens.
#include <algorithm>
#include <climits>
#include <cstring>

#include "mla_internal.h"

namespace mla {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

struct Layout {
  int64_t off_slot, off_items, off_reduce, n_words, off_lse, off_out, total_bytes;
};

Layout layout_for(int64_t slots, int64_t items, int64_t reduce, int64_t partials) {
  Layout l;
  l.off_slot = MLA_PLAN_HEADER_WORDS;
  l.off_items = round_up(l.off_slot + slots + 1, 4);
  l.off_reduce = l.off_items + 4 * items;
  l.n_words = l.off_reduce + 4 * reduce;
  l.off_lse = round_up(4 * l.n_words, kAlignBytes);
  l.off_out = round_up(l.off_lse + 4LL * MLA_NUM_HEADS * partials, kAlignBytes);
  l.total_bytes = l.off_out + 4LL * MLA_NUM_HEADS * MLA_V_DIM * partials;
  return l;
}

}  // namespace

// A plan for at most `total` tokens has at most min(G, ceil(total /
// MIN_CHUNK)) slots, one item per (slot, overlapping sequence) pair (so at
// most slots + batch items), at most two partial items per slot (its first
// and last) and at most one reduce entry per sequence.
DeviceLayout device_layout(int32_t batch, int64_t max_total, int32_t num_cus) {
  const int64_t g = (int64_t)num_cus * MLA_PLAN_WG_PER_CU;
  const int64_t slots = max_total <= 0 ? 0 : std::min<int64_t>(g, ceil_div(max_total, MLA_PLAN_MIN_CHUNK));
  const Layout l = layout_for(slots, slots + batch, batch, 2 * slots);
  return DeviceLayout{slots, l.off_items, l.off_reduce, l.off_lse, l.off_out, l.total_bytes};
}

size_t workspace_bound(int32_t batch, int64_t total, int32_t num_cus) {
  return (size_t)device_layout(batch, total, num_cus).total_bytes;
}

int build_plan(const int32_t* ind, int32_t batch, int32_t num_cus, PlanResult* out,
               std::string* err) {
  if (batch < 0) { *err = "batch must be >= 0"; return MLA_ERR_INVALID; }
  if (num_cus < 1) { *err = "num_cus must be >= 1"; return MLA_ERR_INVALID; }
  if (ind == nullptr) { *err = "kv_indptr is null"; return MLA_ERR_INVALID; }
  if (ind[0] < 0) { *err = "kv_indptr[0] must be >= 0"; return MLA_ERR_INVALID; }
  for (int32_t b = 0; b < batch; ++b) {
    if (ind[b + 1] < ind[b]) { *err = "kv_indptr must be non-decreasing"; return MLA_ERR_INVALID; }
  }
  const int64_t base = ind[0];
  const int64_t end = ind[batch];
  const int64_t total = end - base;
  const int64_t g = (int64_t)num_cus * MLA_PLAN_WG_PER_CU;

  // Item charges: when an equal-token slot (c0) is longer than the fixed
  // work of an item, sequences shorter than c0 share slots, and each of
  // their items costs MLA_PLAN_ITEM_COST tokens' worth besides its tokens.
  // Sequences are laid end to end on a weighted line, a short one taking its
  // charge and then its tokens, and the line is cut into equal slots.
  std::vector<int64_t> start(batch + 1, 0), tok0(batch, 0);
  bool charge = false;
  if (total > 0) {
    const int64_t c0 = std::max<int64_t>(MLA_PLAN_MIN_CHUNK, round_up(ceil_div(total, g), MLA_PLAN_CHUNK_ALIGN));
    charge = c0 > MLA_PLAN_ITEM_COST;
    int64_t pos = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t len = (int64_t)ind[b + 1] - ind[b];
      start[b] = pos;
      tok0[b] = pos + (charge && len > 0 && len < c0 ? MLA_PLAN_ITEM_COST : 0);
      pos = tok0[b] + len;
    }
    start[batch] = pos;
  }
  const int64_t wt = start[batch];
  int64_t chunk = 0, num_slots = 0;
  if (total > 0) {
    chunk = std::max<int64_t>(MLA_PLAN_MIN_CHUNK, round_up(ceil_div(wt, g), MLA_PLAN_CHUNK_ALIGN));
    num_slots = ceil_div(wt, chunk);
  }

  // Items, walking slots in order; a sequence that spans slots gets one
  // partial per piece, numbered consecutively.
  std::vector<int32_t> slot_indptr;
  std::vector<int32_t> items;           // 4 per item
  std::vector<int32_t> n_pieces(batch, 0), first_partial(batch, -1);
  slot_indptr.reserve(num_slots + 1);
  slot_indptr.push_back(0);
  int32_t num_partials = 0;
  int32_t seq = 0;
  for (int64_t s = 0; s < num_slots; ++s) {
    const int64_t lo = s * chunk, hi = (s + 1) * chunk;
    while (seq < batch && start[seq + 1] <= lo) ++seq;
    for (int32_t b = seq; b < batch && start[b] < hi; ++b) {
      // the part of sequence b's tokens inside [lo, hi) on the line
      const int64_t u0 = std::max(lo, tok0[b]), u1 = std::min(hi, start[b + 1]);
      if (u1 <= u0) continue;
      const int64_t sl = ind[b], sh = ind[b + 1];
      const int64_t il = sl + (u0 - tok0[b]), ih = sl + (u1 - tok0[b]);
      int32_t dest = -1;
      if (!(il == sl && ih == sh)) {
        dest = num_partials++;
        if (first_partial[b] < 0) first_partial[b] = dest;
      }
      items.push_back(b);
      items.push_back((int32_t)il);
      items.push_back((int32_t)ih);
      items.push_back(dest);
      ++n_pieces[b];
    }
    slot_indptr.push_back((int32_t)(items.size() / 4));
  }

  std::vector<int32_t> reduce;
  for (int32_t b = 0; b < batch; ++b) {
    if (ind[b + 1] == ind[b]) {
      reduce.insert(reduce.end(), {b, 0, 0, 0});
    } else if (n_pieces[b] >= 2) {
      reduce.insert(reduce.end(), {b, first_partial[b], n_pieces[b], 0});
    }
  }

  const int64_t n_items = (int64_t)items.size() / 4;
  const int64_t n_reduce = (int64_t)reduce.size() / 4;
  const Layout l = layout_for(num_slots, n_items, n_reduce, num_partials);
  if (l.off_out > INT32_MAX) { *err = "plan offsets exceed int32"; return MLA_ERR_INVALID; }

  std::vector<int32_t>& w = out->words;
  w.assign((size_t)l.n_words, 0);
  w[kPwMagic] = MLA_PLAN_MAGIC;
  w[kPwVersion] = MLA_PLAN_VERSION;
  w[kPwBatch] = batch;
  w[kPwBase] = (int32_t)base;
  w[kPwTotal] = (int32_t)total;
  w[kPwNumCus] = num_cus;
  w[kPwChunk] = (int32_t)std::min<int64_t>(chunk, INT32_MAX);   // a record of the rule's value
  w[kPwNumSlots] = (int32_t)num_slots;
  w[kPwNumItems] = (int32_t)n_items;
  w[kPwNumPartials] = num_partials;
  w[kPwNumReduce] = (int32_t)n_reduce;
  w[kPwOffSlot] = (int32_t)l.off_slot;
  w[kPwOffItems] = (int32_t)l.off_items;
  w[kPwOffReduce] = (int32_t)l.off_reduce;
  w[kPwOffLse] = (int32_t)l.off_lse;
  w[kPwOffOut] = (int32_t)l.off_out;
  std::copy(slot_indptr.begin(), slot_indptr.end(), w.begin() + l.off_slot);
  std::copy(items.begin(), items.end(), w.begin() + l.off_items);
  std::copy(reduce.begin(), reduce.end(), w.begin() + l.off_reduce);

  out->workspace_bytes = (size_t)l.total_bytes;
  out->num_slots = (int32_t)num_slots;
  out->num_reduce = (int32_t)n_reduce;
  out->num_partials = num_partials;
  out->off_lse = (int32_t)l.off_lse;
  out->off_out = (int32_t)l.off_out;
  return MLA_OK;
}

}  // namespace mla
