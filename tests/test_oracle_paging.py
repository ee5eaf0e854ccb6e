"""Pins for the oracle's page tables (oracle/paging_ref.py and the
page-table decodes built on it): a hand-worked table, the per-token row
formula, page size 1, identity pages and moved pages reduce to the pinned
contiguous and row-list definitions."""

import numpy as np
import torch

from oracle import dense_ref as dref
from oracle import mxfp4_ref as ref
from oracle import paging_ref as pref

SM = float(np.float32(1.0 / 24.0))


def test_hand_worked_table():
    # page size 4; sequence 0 owns pages 7, 2, 5 with 3 rows in the last,
    # sequence 1 none, sequence 2 page 0 with 4 rows (a full last page)
    rows = pref.page_table_rows([7, 2, 5, 0], [0, 3, 3, 4], [3, 0, 4], 4)
    assert rows[0].tolist() == [28, 29, 30, 31, 8, 9, 10, 11, 20, 21, 22]
    assert rows[1].tolist() == []
    assert rows[2].tolist() == [0, 1, 2, 3]
    assert pref.page_table_token_indptr([0, 3, 3, 4], [3, 0, 4], 4).tolist() == [0, 11, 11, 15]


def test_rows_follow_the_per_token_formula():
    """Token t of a sequence is row pages[t // ps] * ps + t % ps (the
    division form, written independently of the page-by-page expansion)."""
    rng = np.random.default_rng(5)
    for ps in (1, 3, 16, 64):
        npages = rng.integers(0, 5, 6)
        pi = np.concatenate([[0], np.cumsum(npages)])
        pages = rng.permutation(200)[: pi[-1]]
        last = np.where(npages > 0, rng.integers(1, ps + 1, 6), 0)
        rows = pref.page_table_rows(pages, pi, last, ps)
        tok = pref.page_table_token_indptr(pi, last, ps)
        for b in range(6):
            n = int(tok[b + 1] - tok[b])
            want = [int(pages[pi[b] + t // ps]) * ps + t % ps for t in range(n)]
            assert rows[b].tolist() == want


def _rand(rng, rows):
    packed = rng.integers(0, 256, (rows, 288), dtype=np.uint8)
    scales = rng.integers(122, 131, (rows, 18), dtype=np.uint8)
    return packed, scales


def _q(rng, b):
    q = torch.from_numpy(rng.standard_normal((b, 16, 576)).astype(np.float32)).to(torch.bfloat16)
    return q.view(torch.int16).numpy().view(np.uint16)


def test_page_size_one_is_the_row_list():
    rng = np.random.default_rng(6)
    packed, scales = _rand(rng, 40)
    q = _q(rng, 3)
    pi = np.array([0, 5, 5, 12])
    pages = rng.permutation(40)[:12]
    got = ref.mla_decode_ref_page_table(q, packed, scales, pages, pi, [1, 0, 1], 1, SM)
    want = ref.mla_decode_ref_gather(q, packed, scales, pages, pi, SM)
    assert np.array_equal(got, want)


def test_identity_pages_are_the_contiguous_cache():
    """Consecutive pages 0, 1, 2, ... over a contiguous cache, the last one
    partial, give the contiguous definition."""
    rng = np.random.default_rng(7)
    ps = 8
    lens = [19, 8, 1]
    packed, scales = _rand(rng, 64)
    q = _q(rng, 3)
    npages = [(n + ps - 1) // ps for n in lens]
    pi = np.concatenate([[0], np.cumsum(npages)])
    last = [n - (p - 1) * ps for n, p in zip(lens, npages)]
    # sequence b's pages start right after the previous sequence's pages
    pages = np.arange(pi[-1])
    got = ref.mla_decode_ref_page_table(q, packed, scales, pages, pi, last, ps, SM)
    for b, n in enumerate(lens):
        lo = int(pi[b]) * ps
        want = ref.mla_decode_ref(q[b:b + 1], packed[lo:lo + n], scales[lo:lo + n], [0, n], SM)
        assert np.array_equal(got[b], want[0])


def test_moving_pages_in_the_pool_changes_nothing():
    """Moving every page's rows to another page slot and renumbering the
    table leaves all three formats' outputs unchanged; swapping two pages
    of one sequence in its table changes its token order only (a softmax
    over a set: the same value up to rounding)."""
    rng = np.random.default_rng(8)
    ps, slots = 4, 12
    packed, scales = _rand(rng, ps * slots)
    codes = rng.integers(0, 256, (ps * slots, 576), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes
    bits = torch.from_numpy(rng.standard_normal((ps * slots, 576)).astype(np.float32)).to(torch.bfloat16)
    bits = bits.view(torch.int16).numpy().view(np.uint16)
    q = _q(rng, 2)
    pi, last = [0, 3, 5], [2, 4]
    pages = np.array([3, 9, 0, 5, 7])
    perm = rng.permutation(slots)           # page slot s moves to perm[s]
    rowmap = (perm[:, None] * ps + np.arange(ps)).reshape(-1)
    moved = [np.empty_like(a) for a in (packed, scales, codes, bits)]
    for m, a in zip(moved, (packed, scales, codes, bits)):
        m[rowmap] = a
    np.testing.assert_array_equal(
        ref.mla_decode_ref_page_table(q, packed, scales, pages, pi, last, ps, SM),
        ref.mla_decode_ref_page_table(q, moved[0], moved[1], perm[pages], pi, last, ps, SM))
    np.testing.assert_array_equal(
        dref.mla_decode_ref_fp8_page_table(q, codes, 0.5, pages, pi, last, ps, SM),
        dref.mla_decode_ref_fp8_page_table(q, moved[2], 0.5, perm[pages], pi, last, ps, SM))
    np.testing.assert_array_equal(
        dref.mla_decode_ref_bf16_page_table(q, bits, pages, pi, last, ps, SM),
        dref.mla_decode_ref_bf16_page_table(q, moved[3], perm[pages], pi, last, ps, SM))
    # the fp8 / bf16 page-table oracles read the same rows as their row lists
    rows = np.concatenate(pref.page_table_rows(pages, pi, last, ps))
    tok = pref.page_table_token_indptr(pi, last, ps)
    np.testing.assert_array_equal(
        dref.mla_decode_ref_fp8_page_table(q, codes, 0.5, pages, pi, last, ps, SM),
        dref.mla_decode_ref_fp8(q, codes[rows], 0.5, tok, SM))
    np.testing.assert_array_equal(
        dref.mla_decode_ref_bf16_page_table(q, bits, pages, pi, last, ps, SM),
        dref.mla_decode_ref_bf16(q, bits[rows], tok, SM))
    # full pages of sequence 0 in another order: same value up to rounding
    swapped = pages.copy()
    swapped[[0, 1]] = swapped[[1, 0]]
    a = ref.mla_decode_ref_page_table(q, packed, scales, pages, pi, last, ps, SM)
    b = ref.mla_decode_ref_page_table(q, packed, scales, swapped, pi, last, ps, SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
