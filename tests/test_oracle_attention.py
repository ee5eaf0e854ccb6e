"""Pins for the oracle's fp64 attention: brute force, closed forms, invariants."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mxfp4_ref as ref

SM = float(np.float32(1.0 / 24.0))


def _rand_case(rng, lens, q_std=1.0):
    t = sum(lens)
    q = (rng.standard_normal((len(lens), 16, 576)) * q_std).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    qbits = qb.view(torch.int16).numpy().view(np.uint16)
    packed = rng.integers(0, 256, (t, 288), dtype=np.uint8)
    scales = rng.integers(122, 131, (t, 18), dtype=np.uint8)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return qbits, packed, scales, indptr


def _brute(qbits, packed, scales, indptr, sm):
    """Pure-Python definition: element decode from bit fields, exact Fractions
    for every K value, math.fsum dot products, math.exp softmax."""
    def code_val(code):
        s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
        mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
        return -mag if s else mag

    def bf16(bits):
        return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])

    b_n = len(indptr) - 1
    out = np.zeros((b_n, 16, 512))
    s = float(np.float32(sm))
    for b in range(b_n):
        rows = range(int(indptr[b]), int(indptr[b + 1]))
        kv = []
        for t in rows:
            row = []
            for j in range(576):
                byte = int(packed[t, j // 2])
                code = (byte >> 4) if j & 1 else (byte & 15)
                row.append(float(code_val(code) * Fraction(2) ** (int(scales[t, j // 32]) - 127)))
            kv.append(row)
        if not kv:
            continue
        for h in range(16):
            qrow = [bf16(qbits[b, h, j]) for j in range(576)]
            z = [s * math.fsum(qrow[j] * k[j] for j in range(576)) for k in kv]
            zm = max(z)
            e = [math.exp(v - zm) for v in z]
            den = math.fsum(e)
            for d in range(512):
                out[b, h, d] = math.fsum(e[i] * kv[i][d] for i in range(len(kv))) / den
    return out


@pytest.mark.parametrize("lens", [[1], [2, 3], [5, 0, 17]])
def test_bruteforce_tiny(lens):
    rng = np.random.default_rng(sum(lens) + 11)
    qbits, packed, scales, indptr = _rand_case(rng, lens)
    got = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    want = _brute(qbits, packed, scales, indptr, SM)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_matches_torch_float64_attention():
    # library special case: torch's own softmax and matmul in float64 on the
    # exactly dequantised rows
    rng = np.random.default_rng(3)
    lens = [40, 7, 64]
    qbits, packed, scales, indptr = _rand_case(rng, lens, q_std=2.0)
    got = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    q = torch.from_numpy(ref.bf16_bits_to_f64(qbits))
    for b in range(3):
        k = torch.from_numpy(ref.dequant_mxfp4(packed[indptr[b]:indptr[b + 1]],
                                               scales[indptr[b]:indptr[b + 1]]))
        p = torch.softmax((q[b] @ k.T) * SM, dim=-1)
        want = (p @ k[:, :512]).numpy()
        np.testing.assert_allclose(got[b], want, rtol=1e-12, atol=1e-15)


def test_one_token_returns_v_exactly():
    rng = np.random.default_rng(1)
    qbits, packed, scales, indptr = _rand_case(rng, [1, 1])
    got = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    k = ref.dequant_mxfp4(packed, scales)
    for b in range(2):
        for h in range(16):
            assert np.array_equal(got[b, h], k[b, :512])


def test_permutation_invariance():
    rng = np.random.default_rng(2)
    qbits, packed, scales, indptr = _rand_case(rng, [50])
    perm = rng.permutation(50)
    a = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    b = ref.mla_decode_ref(qbits, packed[perm], scales[perm], indptr, SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(4)
    _, packed, scales, indptr = _rand_case(rng, [9])
    qbits = np.zeros((1, 16, 576), np.uint16)
    got = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    k = ref.dequant_mxfp4(packed, scales)
    want = k[:, :512].mean(axis=0)
    for h in range(16):
        np.testing.assert_allclose(got[0, h], want, rtol=1e-13, atol=0)


def test_two_token_closed_form():
    # q has one non-zero element per head (dim 0, value a_h), token 1 has
    # element 0 = 1.0 and token 2 has element 0 = 0, so z1 = sm*a_h, z2 = 0 and
    # out = sigmoid(sm*a_h) v1 + sigmoid(-sm*a_h) v2.
    rng = np.random.default_rng(6)
    packed = rng.integers(0, 256, (2, 288), dtype=np.uint8)  # V dims random
    packed[0, 0] = (packed[0, 0] & 0xF0) | 0x2      # element 0 of token 1 = 1.0
    packed[1, 0] = (packed[1, 0] & 0xF0) | 0x0      # element 0 of token 2 = 0
    scales = np.full((2, 18), 127, np.uint8)
    a = [float(x) for x in np.linspace(-40, 40, 16)]
    qv = torch.zeros(1, 16, 576, dtype=torch.float32)
    for h in range(16):
        qv[0, h, 0] = a[h]
    qb = qv.to(torch.bfloat16)
    a = [float(qb[0, h, 0]) for h in range(16)]
    qbits = qb.view(torch.int16).numpy().view(np.uint16)
    got = ref.mla_decode_ref(qbits, packed, scales, [0, 2], SM)
    k = ref.dequant_mxfp4(packed, scales)
    for h in range(16):
        z = SM * a[h]
        w1 = 1.0 / (1.0 + math.exp(-z))
        w2 = 1.0 / (1.0 + math.exp(z))
        np.testing.assert_allclose(got[0, h], w1 * k[0, :512] + w2 * k[1, :512],
                                   rtol=1e-13, atol=1e-300)


def test_sequences_are_independent():
    rng = np.random.default_rng(7)
    qbits, packed, scales, indptr = _rand_case(rng, [6, 9])
    a = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    p2, s2 = packed.copy(), scales.copy()
    p2[6:] = rng.integers(0, 256, (9, 288), dtype=np.uint8)
    s2[6:] = 124
    b = ref.mla_decode_ref(qbits, p2, s2, indptr, SM)
    assert np.array_equal(a[0], b[0])
    assert not np.allclose(a[1], b[1])


def test_empty_sequence_gives_zeros():
    rng = np.random.default_rng(8)
    qbits, packed, scales, indptr = _rand_case(rng, [0, 3, 0])
    out = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isfinite(out[1]))


def test_nan_scale_poisons_its_sequence_only():
    rng = np.random.default_rng(9)
    qbits, packed, scales, indptr = _rand_case(rng, [4, 4])
    scales[5, 2] = 255
    out = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    assert np.all(np.isfinite(out[0]))
    assert np.all(np.isnan(out[1]))


def test_scale_doubling_equals_query_doubling():
    # z = sm * q.k is bilinear: doubling sm equals doubling q (exact in bf16)
    rng = np.random.default_rng(10)
    qbits, packed, scales, indptr = _rand_case(rng, [12])
    q2 = torch.from_numpy(ref.bf16_bits_to_f64(qbits) * 2).to(torch.bfloat16)
    q2bits = q2.view(torch.int16).numpy().view(np.uint16)
    a = ref.mla_decode_ref(qbits, packed, scales, indptr, 2 * SM)
    b = ref.mla_decode_ref(q2bits, packed, scales, indptr, SM)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-300)
    c = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    assert not np.allclose(a, c)


def test_v_is_first_512_dims_not_rope():
    # changing only the rope part (dims 512..575) of the keys changes the
    # weights but a single token still returns its own first 512 dims
    rng = np.random.default_rng(12)
    qbits, packed, scales, indptr = _rand_case(rng, [1])
    base = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    p2 = packed.copy()
    p2[0, 256:] ^= 0x11
    got = ref.mla_decode_ref(qbits, p2, scales, indptr, SM)
    assert np.array_equal(base, got)


def test_gather_oracle_matches_contiguous():
    """Per-token row lists: identity rows, a permuted pool read through the
    inverse permutation, and rows shared by two sequences all reduce to the
    contiguous definition on the rows actually read."""
    rng = np.random.default_rng(41)
    lens = [3, 0, 7, 2]
    qbits, packed, scales, indptr = _rand_case(rng, lens)
    t = int(indptr[-1])
    want = ref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    ident = np.arange(t, dtype=np.int32)
    assert np.array_equal(ref.mla_decode_ref_gather(qbits, packed, scales, ident, indptr, SM), want)
    # pool of 3t rows: row i of the contiguous cache sits at pool row pos[i]
    pos = rng.permutation(3 * t)[:t].astype(np.int32)
    pool_p = rng.integers(0, 256, (3 * t, 288), dtype=np.uint8)
    pool_s = rng.integers(122, 131, (3 * t, 18), dtype=np.uint8)
    pool_p[pos] = packed
    pool_s[pos] = scales
    assert np.array_equal(ref.mla_decode_ref_gather(qbits, pool_p, pool_s, pos, indptr, SM), want)
    # sequence 3 reads the first two rows of sequence 0 (a shared prefix)
    shared = ident.copy()
    shared[indptr[3]:indptr[4]] = [0, 1]
    got = ref.mla_decode_ref_gather(qbits, packed, scales, shared, indptr, SM)
    copy_p, copy_s = packed.copy(), scales.copy()
    copy_p[indptr[3]:indptr[4]] = packed[0:2]
    copy_s[indptr[3]:indptr[4]] = scales[0:2]
    np.testing.assert_array_equal(got, ref.mla_decode_ref(qbits, copy_p, copy_s, indptr, SM))
    assert not np.array_equal(got[3], want[3])
