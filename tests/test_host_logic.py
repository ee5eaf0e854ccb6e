"""CPU checks of the host-side helpers around the decode: the index guard of
the row-list decodes, the benchmark's byte accounting and the cache byte
counts of the three formats (no GPU)."""

import os
import sys

import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_kv_bytes_per_format():
    assert synth.kv_bytes(1) == 288 + 18
    assert synth.kv_bytes(10, "fp8") == 5760
    assert synth.kv_bytes(10, "bf16") == 11520
    # the cache sizes of 256 sequences of 8192 tokens
    assert synth.kv_bytes(256 * 8192) == 641728512
    assert synth.kv_bytes(256 * 8192, "fp8") == 1207959552
    assert synth.kv_bytes(256 * 8192, "bf16") == 2415919104


def test_algorithmic_bytes():
    import bench
    words = [0] * 16
    words[2] = 256          # batch
    words[9] = 0            # partials
    assert bench.algorithmic_bytes(words, 256 * 8192) == 650641408
    assert bench.algorithmic_bytes(words, 256 * 8192, "fp8") == 1216872448
    assert bench.algorithmic_bytes(words, 256 * 8192, gather=True) == 650641408 + 4 * 256 * 8192
    # through a page table: one 4-byte entry per page, not per token
    assert bench.algorithmic_bytes(words, 256 * 8192, pages=256 * 8192 // 16) == 650641408 + 4 * 256 * 8192 // 16
    words[9] = 3            # each partial written once and read once
    assert bench.algorithmic_bytes(words, 0) - bench.algorithmic_bytes([0] * 16, 0) == \
        256 * bench.QO_BYTES_PER_SEQ + 2 * 3 * 16 * 513 * 4


def test_check_kv_indices():
    ind = [3, 5, 9]                      # tokens 3..8 are read
    idx = torch.arange(12, dtype=torch.int32)
    binding.check_kv_indices(idx, ind, pool_rows=12)
    # entries before kv_indptr[0] are not read, so they may hold anything
    bad_head = idx.clone()
    bad_head[0] = -7
    binding.check_kv_indices(bad_head, ind, pool_rows=12)
    with pytest.raises(ValueError):
        binding.check_kv_indices(idx, ind, pool_rows=8)              # row 8 outside a pool of 8
    with pytest.raises(ValueError):
        neg = idx.clone()
        neg[4] = -1
        binding.check_kv_indices(neg, ind, pool_rows=12)
    with pytest.raises(ValueError):
        binding.check_kv_indices(idx[:8], ind, pool_rows=12)         # shorter than kv_indptr[-1]
    with pytest.raises(ValueError):
        binding.check_kv_indices(idx.to(torch.int64), ind, pool_rows=12)
    with pytest.raises(ValueError):
        binding.check_kv_indices(idx, ind, pool_rows=2 ** 32 // 288 + 1)  # 32-bit row offsets
    binding.check_kv_indices(idx, ind, pool_rows=2 ** 32 // 288)          # the largest pool that fits
    binding.check_kv_indices(idx, [0, 0], pool_rows=1)               # nothing read


def test_fp8_quantiser_edge_cases():
    zeros = torch.zeros(3, 576, dtype=torch.bfloat16)
    codes, scale = synth.quantize_fp8_per_tensor(zeros)
    assert float(scale) == 1.0 and int(codes.max()) == 0
    x = torch.full((2, 576), -2.5, dtype=torch.bfloat16)
    codes, scale = synth.quantize_fp8_per_tensor(x)
    assert torch.all(codes == 0xFE)                                  # -448 after scaling


def test_dense_inputs_share_the_mxfp4_draws():
    w = synth.Workload("t", 2, None, None, 1.0, False, 5)
    q, _, _, ind, _ = synth.make_inputs(w, lengths=[3, 4])
    q2, lat, scale, ind2, _ = synth.make_dense_inputs(w, "bf16", lengths=[3, 4])
    assert torch.equal(q, q2) and torch.equal(ind, ind2) and scale is None
    assert lat.shape == (7, 576) and lat.dtype == torch.bfloat16
    with pytest.raises(ValueError):
        synth.make_dense_inputs(w, "fp4", lengths=[3, 4])


def test_page_table_offsets_and_guards():
    """Token offsets of a page table and the binding's checks of it (host
    only: the checks read CPU tensors just like device ones)."""
    import torch
    from mla_mxfp4_kv_amd import binding
    assert binding.page_table_kv_indptr([0, 3, 3, 4], [3, 0, 4], 4) == [0, 11, 11, 15]
    assert binding.page_table_kv_indptr([2, 2], [0], 16) == [0, 0]
    for pi, last, ps in (([0, 1], [0], 4),      # a page with no rows
                         ([0, 1], [5], 4),      # more rows than the page holds
                         ([0, 2, 1], [1, 1], 4),  # offsets going down
                         ([0, 1], [1], 0)):     # page size 0
        with pytest.raises(ValueError):
            binding.page_table_kv_indptr(pi, last, ps)
    pages = torch.tensor([7, 2, 5, 0], dtype=torch.int32)
    # sequence 0's last page 5 needs rows 20..22, sequence 2's page 0 rows 0..3
    binding.check_page_table(pages, [0, 3, 3, 4], [3, 0, 4], 4, pool_rows=32)
    with pytest.raises(ValueError):   # page 7 (a full page) needs rows up to 31
        binding.check_page_table(pages, [0, 3, 3, 4], [3, 0, 4], 4, pool_rows=31)
    last_page_seven = torch.tensor([2, 7], dtype=torch.int32)
    binding.check_page_table(last_page_seven, [0, 2], [2], 4, pool_rows=30)   # rows 28, 29
    with pytest.raises(ValueError):
        binding.check_page_table(last_page_seven, [0, 2], [3], 4, pool_rows=30)
    with pytest.raises(ValueError):   # negative page
        binding.check_page_table(torch.tensor([-1], dtype=torch.int32), [0, 1], [1], 4, pool_rows=64)
    with pytest.raises(ValueError):   # table shorter than its offsets
        binding.check_page_table(torch.tensor([0], dtype=torch.int32), [0, 2], [1], 4, pool_rows=64)
    with pytest.raises(ValueError):   # wrong dtype
        binding.check_page_table(torch.tensor([0], dtype=torch.int64), [0, 1], [1], 4, pool_rows=64)


def test_grouped_entries_layout():
    """128 heads as 8 groups: entry e = b * 8 + g has sequence b's length and
    starts at its first row; the host planner takes the entries as its
    sequences."""
    entry, starts = binding.group_entries([3, 8, 8, 15], 8)
    assert entry == [0] + [5 * k for k in range(1, 9)] + [40] * 8 + [40 + 7 * k for k in range(1, 9)]
    assert starts == [3] * 8 + [8] * 8 + [8] * 8
    assert binding.group_entries([0, 4], 1) == ([0, 4], [0])
    with pytest.raises(ValueError):
        binding.group_entries([0, 4], 0)
    words, _ = binding.plan_host(entry, 256)
    assert words[2] == 24 and words[4] == 8 * (5 + 7)   # entries and their tokens


def test_page_table_offsets_match_the_oracle():
    """The binding's token offsets of random page tables equal the oracle's,
    and the oracle's page-by-page rows have those lengths."""
    import numpy as np
    from oracle import paging_ref as pref
    rng = np.random.default_rng(0)
    for _ in range(200):
        ps = int(rng.integers(1, 70))
        npages = rng.integers(0, 6, 5)
        pi = np.concatenate([[0], np.cumsum(npages)]).tolist()
        last = [int(rng.integers(1, ps + 1)) if n else 0 for n in npages]
        tok = binding.page_table_kv_indptr(pi, last, ps)
        assert tok == pref.page_table_token_indptr(pi, last, ps).tolist()
        rows = pref.page_table_rows(np.arange(pi[-1]), pi, last, ps)
        assert [len(r) for r in rows] == [b - a for a, b in zip(tok, tok[1:])]
