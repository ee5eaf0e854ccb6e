"""Pins of the 24-scale MXFP4 oracle (oracle.mxfp4_24_ref) to what page
"kernelbot-amd-mixed-mla-717900" fixes (scale k covers elements 24k..24k+23,
i.e. packed bytes 12k..12k+11) and to closed forms of the attention."""

import math

import numpy as np
import pytest

from oracle import mxfp4_24_ref as r24
from oracle import mxfp4_ref as ref

SM = 1.0 / math.sqrt(576.0)


def _rand(t, seed, lo=122, hi=131):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, size=(t, 288), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(t, 24), dtype=np.uint8)
    return rng, packed, scales


def test_hand_worked_block_edge():
    """Bytes 11 and 12 straddle scale blocks 0 and 1: worked by hand."""
    packed = np.zeros((1, 288), dtype=np.uint8)
    scales = np.full((1, 24), 127, dtype=np.uint8)
    packed[0, 11] = 0x72      # element 22: code 2 (1.0); element 23: code 7 (6.0)
    packed[0, 12] = 0x9A      # element 24: code 0xA (-1.0); element 25: code 9 (-0.5)
    scales[0, 0] = 128        # x2
    scales[0, 1] = 125        # x1/4
    v = r24.dequant_mxfp4_24(packed, scales)[0]
    assert v[22] == 2.0 and v[23] == 12.0
    assert v[24] == -0.25 and v[25] == -0.125
    assert np.count_nonzero(v) == 4


def test_byte_wise_statement():
    """Element by element from the byte form of the layout: packed byte j
    holds elements 2j (low nibble) and 2j+1 (high nibble), scaled by byte
    j // 12 of the token's 24."""
    _, packed, scales = _rand(3, 1, lo=100, hi=160)
    got = r24.dequant_mxfp4_24(packed, scales)
    for t in range(3):
        for j in range(288):
            s = 2.0 ** (int(scales[t, j // 12]) - 127)
            lo, hi = int(packed[t, j]) & 15, int(packed[t, j]) >> 4
            assert got[t, 2 * j] == ref.e2m1_value(lo) * s
            assert got[t, 2 * j + 1] == ref.e2m1_value(hi) * s


@pytest.mark.parametrize("k", [0, 5, 21, 23])
def test_nan_byte_spans_one_block(k):
    _, packed, scales = _rand(2, 2)
    scales[1, k] = 255
    v = r24.dequant_mxfp4_24(packed, scales)
    assert not np.isnan(v[0]).any()
    nan = np.flatnonzero(np.isnan(v[1]))
    assert nan.tolist() == list(range(24 * k, 24 * k + 24))


def test_matches_18_scale_layout_when_scales_agree():
    """Scales constant over each 96-element span (4 blocks of 24 = 3 blocks
    of 32) describe the same values in both layouts; the decodes agree."""
    rng, packed, _ = _rand(40, 3)
    span = rng.integers(120, 133, size=(40, 6), dtype=np.uint8)
    s24 = np.repeat(span, 4, axis=1)
    s18 = np.repeat(span, 3, axis=1)
    assert np.array_equal(r24.dequant_mxfp4_24(packed, s24), ref.dequant_mxfp4(packed, s18))
    q = (rng.standard_normal((2, 16, 576)) * 0.5)
    ind = [0, 17, 40]
    np.testing.assert_array_equal(r24.mla_decode_ref_24(q, packed, s24, ind, SM),
                                  ref.mla_decode_ref(q, packed, s18, ind, SM))


def test_layouts_differ_when_blocks_do():
    """A scale change inside a 32-element block that the 24-layout splits is
    visible: element 24 belongs to block 1 in the 24-layout, block 0 in the
    18-layout."""
    packed = np.full((1, 288), 0x22, dtype=np.uint8)   # every element 1.0
    s24 = np.full((1, 24), 127, dtype=np.uint8)
    s24[0, 1] = 130
    v = r24.dequant_mxfp4_24(packed, s24)[0]
    assert v[23] == 1.0 and v[24] == 8.0 and v[47] == 8.0 and v[48] == 1.0


def test_one_token_returns_its_v():
    _, packed, scales = _rand(1, 4)
    q = np.random.default_rng(5).standard_normal((1, 16, 576))
    out = r24.mla_decode_ref_24(q, packed, scales, [0, 1], SM)[0]
    v = r24.dequant_mxfp4_24(packed, scales)[0, :512]
    np.testing.assert_array_equal(out, np.broadcast_to(v, (16, 512)))


def test_two_tokens_logistic_closed_form():
    """Two tokens: the weight of the second is the logistic function of the
    score difference."""
    _, packed, scales = _rand(2, 6)
    q = np.random.default_rng(7).standard_normal((1, 16, 576)) * 0.3
    k = r24.dequant_mxfp4_24(packed, scales)
    out = r24.mla_decode_ref_24(q, packed, scales, [0, 2], SM)[0]
    s = float(np.float32(SM))
    for h in range(16):
        d = s * (float(np.dot(q[0, h], k[1])) - float(np.dot(q[0, h], k[0])))
        w1 = 1.0 / (1.0 + math.exp(-d))
        want = (1.0 - w1) * k[0, :512] + w1 * k[1, :512]
        np.testing.assert_allclose(out[h], want, rtol=1e-12, atol=1e-12)


def test_empty_sequence_and_shape_errors():
    _, packed, scales = _rand(3, 8)
    q = np.ones((2, 16, 576))
    out = r24.mla_decode_ref_24(q, packed, scales, [0, 0, 3], SM)
    assert np.all(out[0] == 0.0) and np.isfinite(out[1]).all()
    with pytest.raises(ValueError):
        r24.dequant_mxfp4_24(packed, scales[:, :18])
    with pytest.raises(ValueError):
        r24.dequant_mxfp4_24(packed[:, :256], scales)
