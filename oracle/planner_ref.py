"""CPU reference planner for the split-K work list.

TEST INFRASTRUCTURE ONLY (see the package docstring). The HIP library has its
own C++ planner; this file is an independent, plain-Python statement of the
same rule, and tests require the two to produce identical int32 words.

Role: the pages build, on the host, a list of work rows
``[batch, partial, q_start, q_end, kv_begin, kv_end, ...]`` plus a per-batch
index of the partials to merge ("kernelbot-amd-mixed-mla-608791", host
metadata builder; "kernelbot-amd-mixed-mla-676098", split heuristic aiming at
about four workgroups per compute unit). The pages split each sequence into
fixed 128-token chunks; the rule here instead cuts the concatenated token
stream into equal contiguous slots, one per workgroup of the device, so that
every workgroup streams about the same number of KV bytes whatever the
length mix, with the fixed work of each item counted in where short
sequences share slots.

The rule (constants in ``PlanConsts``):

* ``T = kv_indptr[B] - kv_indptr[0]``, ``G = num_cus * WG_PER_CU``.
* ``c0 = max(MIN_CHUNK, round_up(ceil(T / G), CHUNK_ALIGN))``: the slot
  length that cuts the token stream alone into equal slots.
* An item costs a fixed amount of work besides its tokens (its Q, its first
  tile in flight, the merge of the workgroup's partial states, its stores),
  about ITEM_COST tokens' worth. When ``c0 > ITEM_COST`` (every workgroup
  has more than that to stream), a sequence with ``0 < len < c0`` is
  *short*: it shares its slot with others, and each such item adds that
  cost. Sequences are laid end to end on a weighted line: sequence b takes
  ``ITEM_COST * short_b + len_b`` units starting at ``W_b`` (``W_0 = 0``),
  the charge first and then its tokens (token ``kv_indptr[b] + j`` at
  ``W_b + ITEM_COST * short_b + j``); ``Wt = W_B``. With no short sequence
  the line is the token stream itself.
* ``chunk = max(MIN_CHUNK, round_up(ceil(Wt / G), CHUNK_ALIGN))`` (at least
  c0, so longer than ITEM_COST whenever a charge exists: no slot lies
  wholly inside one, and every slot owns an item); ``num_slots = ceil(Wt /
  chunk)`` (0 when T is 0). The chunk word stores ``min(chunk, 2^31 - 1)``
  (it records the rule's value; nothing reads it back).
* Slot s owns the units ``[s*chunk, (s+1)*chunk)``; its items are the
  sequences whose tokens meet that range, each cut to it, in ascending b,
  as token ranges ``(b, kv_begin, kv_end, dest)``. Empty sequences give no
  item.
* ``dest = -1`` when the item is the whole sequence (its output is written
  directly); otherwise ``dest`` is the next partial index, so the partials of
  one sequence are consecutive.
* One reduce entry ``(b, first_partial, count, 0)`` per sequence that is
  split (count >= 2) or empty (count 0, meaning "write zeros"), in ascending b.

Word layout (all int32): a 16-word header, ``slot_indptr[num_slots+1]``, the
items (4 words each, starting at a multiple of 4 words), the reduce entries
(4 words each). Then, in the workspace, the partial LSE array (float32
[num_partials, 16]) and the partial output array (float32
[num_partials, 16, 512]) at 256-byte aligned byte offsets recorded in the
header.
"""

from __future__ import annotations

from dataclasses import dataclass, field


class PlanConsts:
    MAGIC = 0x4D4C4134          # 'MLA4'
    VERSION = 1
    HEADER_WORDS = 16
    WG_PER_CU = 1
    CHUNK_ALIGN = 128
    MIN_CHUNK = 256
    ITEM_COST = 512             # fixed work of one item, in tokens
    NUM_HEADS = 16
    V_DIM = 512
    ALIGN_BYTES = 256


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _round_up(a: int, b: int) -> int:
    return _cdiv(a, b) * b


@dataclass
class PlanRef:
    batch: int
    base: int
    total: int
    num_cus: int
    chunk: int
    slot_indptr: list = field(default_factory=list)
    items: list = field(default_factory=list)     # (b, begin, end, dest)
    reduce: list = field(default_factory=list)    # (b, first, count, 0)
    num_partials: int = 0


def build_plan(kv_indptr, batch: int, num_cus: int) -> PlanRef:
    """Apply the slot rule to a host copy of ``kv_indptr`` ([batch+1])."""
    c = PlanConsts
    if batch < 0:
        raise ValueError("batch must be >= 0")
    if num_cus < 1:
        raise ValueError("num_cus must be >= 1")
    ind = [int(v) for v in kv_indptr]
    if len(ind) != batch + 1:
        raise ValueError("kv_indptr must have batch+1 entries")
    if ind[0] < 0:
        raise ValueError("kv_indptr[0] must be >= 0")
    for i in range(batch):
        if ind[i + 1] < ind[i]:
            raise ValueError("kv_indptr must be non-decreasing")
    base, end = ind[0], ind[batch]
    total = end - base
    if end >= 2**31:
        raise ValueError("token count must stay below 2^31")

    g = num_cus * c.WG_PER_CU
    lens = [ind[i + 1] - ind[i] for i in range(batch)]
    short = [0] * batch
    if total:
        c0 = max(c.MIN_CHUNK, _round_up(_cdiv(total, g), c.CHUNK_ALIGN))
        if c0 > c.ITEM_COST:
            short = [1 if 0 < n < c0 else 0 for n in lens]
    # the weighted line: start of each sequence and start of its tokens
    starts, tok0 = [], []
    pos = 0
    for i in range(batch):
        starts.append(pos)
        tok0.append(pos + c.ITEM_COST * short[i])
        pos = tok0[-1] + lens[i]
    starts.append(pos)
    wt = pos
    chunk, num_slots = 0, 0
    if total:
        chunk = max(c.MIN_CHUNK, _round_up(_cdiv(wt, g), c.CHUNK_ALIGN))
        num_slots = _cdiv(wt, chunk)

    plan = PlanRef(batch=batch, base=base, total=total, num_cus=num_cus,
                   chunk=min(chunk, 2 ** 31 - 1))
    plan.slot_indptr.append(0)
    pieces = {}                      # b -> number of items
    first_partial = {}
    for s in range(num_slots):
        lo, hi = s * chunk, (s + 1) * chunk
        for bb in range(batch):
            # the part of sequence bb's tokens inside [lo, hi), on the line
            u0, u1 = max(lo, tok0[bb]), min(hi, starts[bb + 1])
            if u1 <= u0:
                continue
            it_lo = ind[bb] + (u0 - tok0[bb])
            it_hi = ind[bb] + (u1 - tok0[bb])
            if it_lo == ind[bb] and it_hi == ind[bb + 1]:
                dest = -1
            else:
                dest = plan.num_partials
                plan.num_partials += 1
                first_partial.setdefault(bb, dest)
            plan.items.append((bb, it_lo, it_hi, dest))
            pieces[bb] = pieces.get(bb, 0) + 1
        plan.slot_indptr.append(len(plan.items))

    for bi in range(batch):
        if ind[bi + 1] == ind[bi]:
            plan.reduce.append((bi, 0, 0, 0))
        elif pieces.get(bi, 0) >= 2:
            first = first_partial[bi]
            plan.reduce.append((bi, first, pieces[bi], 0))
    return plan


def _layout(num_slots: int, num_items: int, num_reduce: int, num_partials: int):
    c = PlanConsts
    off_slot = c.HEADER_WORDS
    off_items = _round_up(off_slot + num_slots + 1, 4)
    off_reduce = off_items + 4 * num_items
    n_words = off_reduce + 4 * num_reduce
    off_lse = _round_up(4 * n_words, c.ALIGN_BYTES)
    off_o = _round_up(off_lse + 4 * c.NUM_HEADS * num_partials, c.ALIGN_BYTES)
    total_bytes = off_o + 4 * c.NUM_HEADS * c.V_DIM * num_partials
    return off_slot, off_items, off_reduce, n_words, off_lse, off_o, total_bytes


def plan_words_ref(kv_indptr, batch: int, num_cus: int):
    """Return ``(words, workspace_bytes_needed)`` for the plan of ``kv_indptr``."""
    c = PlanConsts
    p = build_plan(kv_indptr, batch, num_cus)
    num_slots = len(p.slot_indptr) - 1
    (off_slot, off_items, off_reduce, n_words,
     off_lse, off_o, need) = _layout(num_slots, len(p.items), len(p.reduce), p.num_partials)
    if off_o >= 2**31:
        raise ValueError("plan offsets exceed int32")
    w = [0] * n_words
    w[0] = c.MAGIC
    w[1] = c.VERSION
    w[2] = batch
    w[3] = p.base
    w[4] = p.total
    w[5] = num_cus
    w[6] = p.chunk
    w[7] = num_slots
    w[8] = len(p.items)
    w[9] = p.num_partials
    w[10] = len(p.reduce)
    w[11] = off_slot
    w[12] = off_items
    w[13] = off_reduce
    w[14] = off_lse
    w[15] = off_o
    for i, v in enumerate(p.slot_indptr):
        w[off_slot + i] = v
    for i, it in enumerate(p.items):
        w[off_items + 4 * i: off_items + 4 * i + 4] = list(it)
    for i, r in enumerate(p.reduce):
        w[off_reduce + 4 * i: off_reduce + 4 * i + 4] = list(r)
    return w, need


def decode_plan_words(words):
    """Parse plan words back into a dict (for invariant checks in tests)."""
    h = list(words[:PlanConsts.HEADER_WORDS])
    num_slots, num_items, num_reduce = h[7], h[8], h[10]
    off_slot, off_items, off_reduce = h[11], h[12], h[13]
    slot = list(words[off_slot: off_slot + num_slots + 1])
    items = [tuple(words[off_items + 4 * i: off_items + 4 * i + 4]) for i in range(num_items)]
    red = [tuple(words[off_reduce + 4 * i: off_reduce + 4 * i + 4]) for i in range(num_reduce)]
    return {
        "magic": h[0], "version": h[1], "batch": h[2], "base": h[3], "total": h[4],
        "num_cus": h[5], "chunk": h[6], "num_slots": num_slots, "num_items": num_items,
        "num_partials": h[9], "num_reduce": num_reduce, "off_lse": h[14], "off_o": h[15],
        "slot_indptr": slot, "items": items, "reduce": red,
    }


def workspace_bound_ref(batch: int, total: int, num_cus: int) -> int:
    """Upper bound on the workspace bytes for any indptr with these sizes."""
    c = PlanConsts
    g = num_cus * c.WG_PER_CU
    if total <= 0:
        slots = 0
    else:
        # short sequences exist only when a slot is longer than ITEM_COST,
        # so the charges never shorten a slot below that (nor MIN_CHUNK)
        slots = min(g, _cdiv(total, c.MIN_CHUNK))
    items = slots + batch
    partials = 2 * slots
    reduce = batch
    return _layout(slots, items, reduce, partials)[6]
