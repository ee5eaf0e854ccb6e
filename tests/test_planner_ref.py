"""Pins for the CPU reference planner: hand-worked plans and invariants."""

import random

import pytest

from oracle.planner_ref import (PlanConsts, build_plan, decode_plan_words,
                                plan_words_ref, workspace_bound_ref)


def test_hand_worked_plan_two_cus():
    # indptr [0, 300, 300, 700]: T = 700, G = 2 -> ceil(700/2)=350 -> round up
    # to 384 (multiple of 128, >= 256). Slots: [0,384) and [384,700).
    # Slot 0: seq 0 whole [0,300) direct; seq 2 part [300,384) -> partial 0.
    # Slot 1: seq 2 part [384,700) -> partial 1.
    # Reduce: seq 1 empty -> (1,0,0,0); seq 2 split -> (2,0,2,0).
    words, need = plan_words_ref([0, 300, 300, 700], 3, 2)
    hdr = [PlanConsts.MAGIC, 1, 3, 0, 700, 2, 384, 2, 3, 2, 2, 16, 20, 32]
    assert words[:14] == hdr
    assert words[16:19] == [0, 2, 3]
    assert words[20:32] == [0, 0, 300, -1, 2, 300, 384, 0, 2, 384, 700, 1]
    assert words[32:40] == [1, 0, 0, 0, 2, 0, 2, 0]
    assert len(words) == 40
    assert words[14] == 256                   # 160 bytes of words -> next 256
    assert words[15] == 256 + 256             # 2 partials * 64 B lse -> 256
    assert need == 512 + 2 * 16 * 512 * 4


def test_hand_worked_plan_with_item_charges():
    # lens [3000, 200, 100, 700] on 2 CUs: T = 4000, ceil(4000/2) = 2000 ->
    # c0 = 2048 > ITEM_COST = 512, so the sequences shorter than 2048 (b = 1,
    # 2, 3) are short and each carries 512 units ahead of its tokens.
    # Line: seq 0 tokens [0,3000); seq 1 charge [3000,3512), tokens
    # [3512,3712); seq 2 charge [3712,4224), tokens [4224,4324); seq 3 charge
    # [4324,4836), tokens [4836,5536). Wt = 5536 -> ceil(5536/2) = 2768 ->
    # chunk 2816, 2 slots: [0,2816) and [2816,5632).
    # Slot 0: seq 0 tokens [0,2816) -> partial 0.
    # Slot 1: seq 0 [2816,3000) -> partial 1; seqs 1, 2, 3 whole.
    # (The equal-token cut would give slot 1 the 952 tokens left of seq 0
    # plus all three short sequences: four items against one.)
    words, need = plan_words_ref([0, 3000, 3200, 3300, 4000], 4, 2)
    hdr = [PlanConsts.MAGIC, 1, 4, 0, 4000, 2, 2816, 2, 5, 2, 1, 16, 20, 40]
    assert words[:14] == hdr
    assert words[16:19] == [0, 1, 5]
    assert words[20:40] == [0, 0, 2816, 0, 0, 2816, 3000, 1, 1, 3000, 3200, -1,
                            2, 3200, 3300, -1, 3, 3300, 4000, -1]
    assert words[40:44] == [0, 0, 2, 0]
    assert len(words) == 44
    assert words[14] == 256 and words[15] == 512
    assert need == 512 + 2 * 16 * 512 * 4


def test_b256_kv8192_is_one_sequence_per_slot():
    ind = [8192 * i for i in range(257)]
    d = decode_plan_words(plan_words_ref(ind, 256, 256)[0])
    assert d["chunk"] == 8192 and d["num_slots"] == 256
    assert d["num_partials"] == 0 and d["num_reduce"] == 0
    assert d["items"] == [(b, 8192 * b, 8192 * (b + 1), -1) for b in range(256)]


def test_long_single_sequence_splits_evenly():
    d = decode_plan_words(plan_words_ref([0, 65536], 1, 256)[0])
    assert d["chunk"] == 256 and d["num_slots"] == 256
    assert d["num_partials"] == 256
    assert d["reduce"] == [(0, 0, 256, 0)]


def test_empty_batch_and_all_empty():
    w, need = plan_words_ref([0], 0, 8)
    d = decode_plan_words(w)
    assert d["num_slots"] == 0 and d["num_items"] == 0 and d["num_reduce"] == 0
    d = decode_plan_words(plan_words_ref([5, 5, 5], 2, 8)[0])
    assert d["base"] == 5 and d["total"] == 0
    assert d["reduce"] == [(0, 0, 0, 0), (1, 0, 0, 0)]


def test_rejects_bad_indptr():
    with pytest.raises(ValueError):
        build_plan([0, 5, 3], 2, 4)
    with pytest.raises(ValueError):
        build_plan([-1, 5], 1, 4)
    with pytest.raises(ValueError):
        build_plan([0, 5], 2, 4)
    with pytest.raises(ValueError):
        build_plan([0, 5], 1, 0)


def _check_invariants(ind, num_cus):
    b_n = len(ind) - 1
    words, need = plan_words_ref(ind, b_n, num_cus)
    d = decode_plan_words(words)
    base, end = ind[0], ind[-1]
    total = end - base
    chunk = d["chunk"]
    assert need <= workspace_bound_ref(b_n, total, num_cus)
    # which sequences carry the item charge (only when an equal-token slot is
    # longer than the charge)
    g = num_cus * PlanConsts.WG_PER_CU
    c0 = max(PlanConsts.MIN_CHUNK, -(-(-(-total // g)) // PlanConsts.CHUNK_ALIGN) * PlanConsts.CHUNK_ALIGN)
    lens = [ind[b + 1] - ind[b] for b in range(b_n)]
    charged = [total > 0 and c0 > PlanConsts.ITEM_COST and 0 < n < c0 for n in lens]
    if total:
        assert chunk >= max(PlanConsts.MIN_CHUNK, c0 if any(charged) else 0)
        assert chunk % PlanConsts.CHUNK_ALIGN == 0
        assert d["num_slots"] <= g
    flat = []
    pieces = {}
    for s in range(d["num_slots"]):
        its = d["items"][d["slot_indptr"][s]:d["slot_indptr"][s + 1]]
        assert its, "every slot owns at least one item"
        for a, c in zip(its, its[1:]):
            assert a[2] == c[1] and a[0] < c[0]
        # a slot holds chunk units of the weighted line: its tokens plus the
        # charges of the short sequences that start in it, give or take less
        # than one charge cut by each edge
        load = sum(ke - kb + PlanConsts.ITEM_COST * (charged[b] and kb == ind[b]) for (b, kb, ke, _) in its)
        assert load < chunk + PlanConsts.ITEM_COST
        if s < d["num_slots"] - 1:
            assert load > chunk - PlanConsts.ITEM_COST
            if not any(charged):
                assert load == chunk
        for (b, kb, ke, dest) in its:
            assert ind[b] <= kb < ke <= ind[b + 1]
            assert (dest == -1) == (kb == ind[b] and ke == ind[b + 1])
            flat.append((kb, ke))
            pieces.setdefault(b, []).append(dest)
    # slots in order cover the token stream in order, without gaps
    pos = base
    for kb, ke in flat:
        assert kb == pos
        pos = ke
    assert pos == end
    partial_ids = sorted(x for v in pieces.values() for x in v if x >= 0)
    assert partial_ids == list(range(d["num_partials"]))
    assert d["num_partials"] <= 2 * d["num_slots"]
    red = {r[0]: r for r in d["reduce"]}
    assert [r[0] for r in d["reduce"]] == sorted(red)
    for b in range(b_n):
        if ind[b + 1] == ind[b]:
            assert red[b] == (b, 0, 0, 0)
        elif len(pieces[b]) >= 2:
            first = red[b][1]
            assert pieces[b] == list(range(first, first + len(pieces[b])))
            assert red[b][2] == len(pieces[b])
        else:
            assert b not in red and pieces[b] == [-1]


def test_invariants_random():
    rng = random.Random(0)
    for trial in range(300):
        b_n = rng.randint(0, 40)
        base = rng.choice([0, 0, 0, rng.randint(0, 1000)])
        ind = [base]
        for _ in range(b_n):
            ind.append(ind[-1] + rng.choice([0, 1, 2, rng.randint(0, 300), rng.randint(0, 5000)]))
        _check_invariants(ind, rng.choice([1, 2, 3, 7, 64, 256, 304]))


def test_invariants_workload_shapes():
    from mla_mxfp4_kv_amd import synth
    for name, w in synth.WORKLOADS.items():
        lens = synth.seq_lengths(w)
        ind = [0]
        for n in lens:
            ind.append(ind[-1] + n)
        for cus in (1, 7, 64, 256):
            _check_invariants(ind, cus)
