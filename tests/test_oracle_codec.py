"""Pins for the oracle's MXFP4 decoding (value tables, layout, exactness)."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import mxfp4_ref as ref


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _e2m1_arith(code):
    """The e2m1 value from its bit fields s|e1 e0|m: subnormal m/2 when the
    exponent field is 0, else (1 + m/2) * 2^(e-1); the sign bit negates.
    (Arithmetic statement on page "kernelbot-amd-mixed-mla-717900",
    ``_nibble_to_f32``.)"""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -mag if s else mag


def test_e2m1_table_matches_golden(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e2m1_values.txt"))
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s), float(val_s)
        got = ref.e2m1_value(code)
        assert got == val
        assert math.copysign(1.0, got) == math.copysign(1.0, val)  # -0 for code 8


def test_e2m1_table_matches_bitfield_formula():
    # the two page statements of the same code table agree on all 16 codes
    for code in range(16):
        assert Fraction(ref.e2m1_value(code)) == _e2m1_arith(code)


def test_e8m0_matches_golden(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e8m0_values.txt"))
    for row in rows:
        byte = int(row[0])
        got = float(ref.e8m0_scale(byte))
        if row[1] == "nan":
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, int(row[2]))


def test_e8m0_all_bytes_are_powers_of_two():
    b = np.arange(255)
    s = ref.e8m0_scale(b)
    m, e = np.frexp(s)
    assert np.all(m == 0.5)
    assert np.array_equal(e - 1, b - 127)


def test_dequant_layout_hand_example():
    packed = np.zeros((2, 288), np.uint8)
    scales = np.full((2, 18), 127, np.uint8)
    packed[0, 0] = 0x71            # element 0 = code 1 (0.5), element 1 = code 7 (6.0)
    packed[0, 15] = 0x9A           # elements 30, 31: code 10 (-1.0), code 9 (-0.5)
    packed[0, 16] = 0x2F           # elements 32, 33: code 15 (-6.0), code 2 (1.0)
    packed[1, 287] = 0x53          # elements 574, 575: code 3 (1.5), code 5 (3.0)
    scales[0, 0] = 129             # block 0 -> x4
    scales[0, 1] = 125             # block 1 -> x1/4
    scales[1, 17] = 130            # block 17 -> x8
    k = ref.dequant_mxfp4(packed, scales)
    assert k.shape == (2, 576)
    assert k[0, 0] == 0.5 * 4 and k[0, 1] == 6.0 * 4
    assert k[0, 30] == -1.0 * 4 and k[0, 31] == -0.5 * 4
    assert k[0, 32] == -6.0 / 4 and k[0, 33] == 1.0 / 4
    assert k[1, 574] == 1.5 * 8 and k[1, 575] == 3.0 * 8
    nz = np.count_nonzero(k)
    assert nz == 8


def test_dequant_bruteforce_fraction():
    rng = np.random.default_rng(5)
    packed = rng.integers(0, 256, (3, 288), dtype=np.uint8)
    scales = rng.integers(1, 255, (3, 18), dtype=np.uint8)
    k = ref.dequant_mxfp4(packed, scales)
    for t in range(3):
        for j in range(576):
            byte = int(packed[t, j // 2])
            code = (byte >> 4) if (j % 2) else (byte & 0xF)
            want = _e2m1_arith(code) * Fraction(2) ** (int(scales[t, j // 32]) - 127)
            assert Fraction(k[t, j]) == want


def test_dequant_e8m0_255_is_nan_and_0_is_tiny():
    packed = np.full((1, 288), 0x11, np.uint8)   # every element 0.5
    scales = np.full((1, 18), 127, np.uint8)
    scales[0, 3] = 255
    scales[0, 4] = 0
    k = ref.dequant_mxfp4(packed, scales)
    assert np.all(np.isnan(k[0, 96:128]))
    assert np.all(k[0, 128:160] == math.ldexp(0.5, -127))
    assert np.all(k[0, :96] == 0.5)


def test_bf16_bits_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    v = ref.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0
    assert v[2] == 3.140625
    assert v[3] == math.ldexp(1.0, -133)
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127
    assert v[5] == 0.0 and math.copysign(1, v[6]) == -1


def test_shape_checks():
    with pytest.raises(ValueError):
        ref.dequant_mxfp4(np.zeros((1, 287), np.uint8), np.zeros((1, 18), np.uint8))
    with pytest.raises(ValueError):
        ref.dequant_mxfp4(np.zeros((1, 288), np.uint8), np.zeros((1, 24), np.uint8))
