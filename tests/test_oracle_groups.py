"""Pins for the oracle of query entries that share their sequence's rows
(q_seq_len > 1, 128 heads as 8 groups of 16): a closed form for the
entry -> sequence mapping, the single-group case, a duplicated-cache
formulation and head-permutation covariance."""

import numpy as np
import torch

from oracle import dense_ref as dref
from oracle import mxfp4_ref as ref

SM = float(np.float32(1.0 / 24.0))


def _q(rng, e):
    q = torch.from_numpy(rng.standard_normal((e, 16, 576)).astype(np.float32)).to(torch.bfloat16)
    return q.view(torch.int16).numpy().view(np.uint16)


def _cache(rng, t):
    return (rng.integers(0, 256, (t, 288), dtype=np.uint8), rng.integers(122, 131, (t, 18), dtype=np.uint8))


def test_entries_read_their_own_sequence():
    """Every row of a sequence identical: softmax weights sum to one, so
    each entry's output is exactly its sequence's V row. With q_seq_len = 2
    entries 0, 1 belong to sequence 0 and entries 2, 3 to sequence 1 (the
    Triton decode's batch = token // q_seq_len)."""
    rng = np.random.default_rng(1)
    row_a, row_b = _cache(rng, 1), _cache(rng, 1)
    packed = np.concatenate([np.repeat(row_a[0], 5, 0), np.repeat(row_b[0], 3, 0)])
    scales = np.concatenate([np.repeat(row_a[1], 5, 0), np.repeat(row_b[1], 3, 0)])
    got = ref.mla_decode_ref_groups(_q(rng, 4), packed, scales, [0, 5, 8], 2, SM)
    va = ref.dequant_mxfp4(row_a[0], row_a[1])[0, :512]
    vb = ref.dequant_mxfp4(row_b[0], row_b[1])[0, :512]
    for e, v in ((0, va), (1, va), (2, vb), (3, vb)):
        np.testing.assert_allclose(got[e], np.broadcast_to(v, (16, 512)), rtol=1e-13, atol=1e-13)
    assert not np.allclose(va, vb)


def test_one_group_is_the_plain_decode():
    rng = np.random.default_rng(2)
    packed, scales = _cache(rng, 9)
    q = _q(rng, 3)
    ind = [0, 2, 2, 9]
    np.testing.assert_array_equal(ref.mla_decode_ref_groups(q, packed, scales, ind, 1, SM),
                                  ref.mla_decode_ref(q, packed, scales, ind, SM))


def test_groups_equal_a_duplicated_cache():
    """Sharing rows equals giving every entry its own copy of them, for all
    three cache formats."""
    rng = np.random.default_rng(3)
    lens, g = [4, 0, 6], 3
    ind = np.concatenate([[0], np.cumsum(lens)])
    packed, scales = _cache(rng, int(ind[-1]))
    codes = rng.integers(0, 0x7E, (int(ind[-1]), 576), dtype=np.uint8)
    bits = torch.from_numpy(rng.standard_normal((int(ind[-1]), 576)).astype(np.float32)).to(torch.bfloat16)
    bits = bits.view(torch.int16).numpy().view(np.uint16)
    q = _q(rng, len(lens) * g)
    rows = np.concatenate([np.arange(ind[e // g], ind[e // g + 1]) for e in range(len(lens) * g)])
    dup_ind = np.concatenate([[0], np.cumsum([lens[e // g] for e in range(len(lens) * g)])])
    np.testing.assert_array_equal(ref.mla_decode_ref_groups(q, packed, scales, ind, g, SM),
                                  ref.mla_decode_ref(q, packed[rows], scales[rows], dup_ind, SM))
    np.testing.assert_array_equal(dref.mla_decode_ref_fp8_groups(q, codes, 0.25, ind, g, SM),
                                  dref.mla_decode_ref_fp8(q, codes[rows], 0.25, dup_ind, SM))
    np.testing.assert_array_equal(dref.mla_decode_ref_bf16_groups(q, bits, ind, g, SM),
                                  dref.mla_decode_ref_bf16(q, bits[rows], dup_ind, SM))


def test_128_heads_permute_with_their_query():
    """128 heads as 8 groups of 16: permuting the heads of a sequence's
    query permutes its output rows the same way."""
    rng = np.random.default_rng(4)
    packed, scales = _cache(rng, 7)
    ind = [0, 3, 7]
    q = _q(rng, 16).reshape(2, 128, 576)
    perm = rng.permutation(128)
    a = ref.mla_decode_ref_groups(q.reshape(16, 16, 576), packed, scales, ind, 8, SM).reshape(2, 128, 512)
    b = ref.mla_decode_ref_groups(q[:, perm].reshape(16, 16, 576), packed, scales, ind, 8, SM).reshape(2, 128, 512)
    np.testing.assert_allclose(b, a[:, perm], rtol=1e-13, atol=1e-13)
