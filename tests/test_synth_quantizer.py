"""Pins for the MXFP4 encoder that builds the synthetic caches.

Worked examples are derived by hand from the encoding rule (shared exponent
floor(log2 amax) - 2, round to nearest e2m1 with ties to even, saturate at 6).
"""

import math

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import synth
from oracle import mxfp4_ref as ref


def _block(values, fill=0.0):
    x = torch.full((1, 576), fill, dtype=torch.float64)
    for i, v in enumerate(values):
        x[0, i] = v
    return x


def _codes(packed):
    p = packed.numpy()
    c = np.empty((p.shape[0], 576), np.uint8)
    c[:, 0::2] = p & 15
    c[:, 1::2] = p >> 4
    return c


def test_worked_example_amax_3_7():
    # amax 3.7 -> floor(log2) = 1 -> E = -1 -> byte 126; x / 2^-1 = 2x
    x = _block([3.7, 1.3, -0.625, 0.2])
    packed, scales = synth.quantize_mxfp4(x)
    assert int(scales[0, 0]) == 126
    c = _codes(packed)[0]
    assert c[0] == 7        # 7.4 saturates to 6  -> 3.0
    assert c[1] == 5        # 2.6 -> 3            -> 1.5
    assert c[2] == 8 | 2    # -1.25 ties to -1    -> -0.5
    assert c[3] == 1        # 0.4 -> 0.5          -> 0.25
    k = ref.dequant_mxfp4(packed.numpy(), scales.numpy())
    assert list(k[0, :4]) == [3.0, 1.5, -0.5, 0.25]


@pytest.mark.parametrize("y,code", [
    (0.25, 0), (0.2500001, 1), (0.75, 2), (0.7499999, 1), (1.25, 2), (1.2500001, 3),
    (1.75, 4), (2.5, 4), (2.5000001, 5), (3.5, 6), (3.4999999, 5), (5.0, 6),
    (5.0000001, 7), (6.0, 7), (7.9, 7),
])
def test_ties_to_even_and_saturation(y, code):
    # amax pinned to 4 (E = 0, byte 127) by element 31, so x == y
    x = _block([y], 0.0)
    x[0, 31] = 4.0
    packed, scales = synth.quantize_mxfp4(x)
    assert int(scales[0, 0]) == 127
    assert _codes(packed)[0, 0] == code


def test_all_zero_block_and_negative_sign():
    x = _block([-0.1, 0.0], 0.0)
    x[0, 32:64] = 0.0
    x[0, 40] = -3.0
    x[0, 0:32] = 0.0
    x[0, 0] = 0.0
    packed, scales = synth.quantize_mxfp4(x)
    assert int(scales[0, 0]) == 127                # all-zero block
    assert np.all(_codes(packed)[0, :32] == 0)
    assert int(scales[0, 1]) == 127 + 1 - 2        # amax 3 -> floor(log2)=1 -> E=-1
    assert _codes(packed)[0, 40] == 8 | 7          # -6 at E=-1 -> -3.0


def test_grid_values_round_trip_exactly():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(0)
    for e in (-5, -1, 0, 3):
        vals = rng.choice(grid, 576) * rng.choice([-1, 1], 576)
        vals[::32] = 6.0             # amax 6 -> floor(log2 6) = 2 -> E = 0
        x = torch.from_numpy(vals * 2.0 ** e).reshape(1, 576)
        packed, scales = synth.quantize_mxfp4(x)
        assert np.all(scales.numpy() == 127 + e)
        k = ref.dequant_mxfp4(packed.numpy(), scales.numpy())
        np.testing.assert_array_equal(k[0], vals * 2.0 ** e)


def test_error_bound_on_random_rows():
    # outside saturation the encoder error is at most half a grid step
    g = torch.Generator().manual_seed(3)
    x = torch.randn(64, 576, generator=g).to(torch.bfloat16).to(torch.float64)
    packed, scales = synth.quantize_mxfp4(x)
    k = ref.dequant_mxfp4(packed.numpy(), scales.numpy())
    xs = x.numpy()
    sc = ref.e8m0_scale(scales.numpy()).repeat(32, axis=1)
    y = np.abs(xs / sc)
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(k - xs) / sc
    unsat = y <= 6
    assert np.all(err[unsat] <= step[unsat] / 2 + 1e-12)
    assert np.all(np.abs(k[~unsat]) == 6 * sc[~unsat])


def test_make_inputs_shapes_and_determinism():
    w = synth.Workload("t", 3, None, (5, 40), 2.0, True, 7)
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    q, packed, scales, indptr, lens = a
    assert q.shape == (3, 16, 576) and q.dtype == torch.bfloat16
    assert packed.shape == (sum(lens), 288) and scales.shape == (sum(lens), 18)
    assert indptr.tolist() == [0, lens[0], lens[0] + lens[1], sum(lens)]
    assert all(5 <= n <= 40 for n in lens)
    for u, v in zip(a[:4], b[:4]):
        assert torch.equal(u, v)
    assert synth.kv_bytes(10) == 3060


def test_workload_table():
    w = synth.WORKLOADS
    assert synth.seq_lengths(w["b256_kv8192"]) == [8192] * 256
    r = synth.seq_lengths(w["b128_ragged"])
    assert len(r) == 128 and min(r) >= 256 and max(r) <= 32768
    assert math.isclose(w["b4_kv1024"].sm_scale, 1 / 24)


def test_24_element_blocks_follow_the_32_element_rule():
    """quantize_mxfp4(x, 24) applies the same per-block rule to 24-element
    blocks: each block, placed alone in the first 32-element block of an
    otherwise zero row (zeros change no block max), gets the same codes and
    scale byte from the already-pinned 32-element encoding."""
    from mla_mxfp4_kv_amd import synth
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(6, 576, generator=g) * torch.exp2(torch.randint(-6, 7, (6, 1), generator=g).float()))
    x[1, 24:48] = 0.0                     # an all-zero block
    x = x.to(torch.bfloat16)
    pk24, sc24 = synth.quantize_mxfp4(x, 24)
    assert pk24.shape == (6, 288) and sc24.shape == (6, 24)
    codes24 = torch.stack([pk24 & 15, pk24 >> 4], dim=2).reshape(6, 576)
    for t in range(6):
        for k in range(24):
            row = torch.zeros(1, 576, dtype=torch.bfloat16)
            row[0, :24] = x[t, 24 * k:24 * k + 24]
            pk32, sc32 = synth.quantize_mxfp4(row, 32)
            codes32 = torch.stack([pk32 & 15, pk32 >> 4], dim=2).reshape(576)
            assert int(sc24[t, k]) == int(sc32[0, 0]), (t, k)
            assert torch.equal(codes24[t, 24 * k:24 * k + 24], codes32[:24]), (t, k)
    assert int(sc24[1, 1]) == 127 and int(codes24[1, 24:48].max()) == 0
