"""Pins for the oracle of the fp8 (e4m3 + per-tensor scale) and bf16 KV
caches: value tables, library conversions, brute force, cross-format
agreement with the MXFP4 oracle, closed forms and scale wiring."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import synth
from oracle import dense_ref as dref
from oracle import mxfp4_ref as mref

SM = float(np.float32(1.0 / 24.0))


def _table(path):
    with open(path) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _qbits(rng, b, std=1.0):
    q = torch.from_numpy((rng.standard_normal((b, 16, 576)) * std).astype(np.float32))
    return q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3_matches_golden(golden_dir):
    rows = _table(os.path.join(golden_dir, "e4m3_values.txt"))
    assert len(rows) >= 20
    for code_s, val_s in rows:
        got = dref.e4m3_value(int(code_s, 16))
        if val_s == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val_s)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val_s))


def test_e4m3_all_codes_match_torch_float8():
    # torch's float8_e4m3fn widening is an independent statement of the format
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    lib = lib.to(torch.float64).numpy()
    mine = dref.E4M3_VALUES
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(mine))
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(lib[~nan], mine[~nan])
    assert np.array_equal(np.signbit(lib[~nan]), np.signbit(mine[~nan]))
    assert np.nanmax(mine) == dref.FP8_MAX == 448.0


def test_e4m3_structure():
    v = dref.E4M3_VALUES
    # sign symmetry, monotone magnitudes over the positive finite codes
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    pos = v[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)
    # subnormal spacing 2^-9, then each binade has 8 steps of 2^(e-10)
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)
    for e in range(1, 15):
        seg = pos[8 * e:8 * e + 8]
        assert np.all(np.diff(seg) == 2.0 ** (e - 10))


def test_bf16_dequant_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, (7, 576), dtype=np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = dref.dequant_bf16(bits)
    same = np.isnan(lib) == np.isnan(mine)
    assert np.all(same)
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], mine[ok])


def _brute_fp8(qbits, codes, kv_scale, indptr, sm):
    """Pure-Python definition: e4m3 codes from bit fields as Fractions, times
    the float32 scale, math.fsum dot products, math.exp softmax."""
    def val(c):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        return -mag if s else mag

    def bf16(b):
        return float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])

    sc = Fraction(float(np.float32(kv_scale)))
    s = float(np.float32(sm))
    out = np.zeros((len(indptr) - 1, 16, 512))
    for b in range(len(indptr) - 1):
        k = [[float(val(int(c)) * sc) for c in codes[t]] for t in range(indptr[b], indptr[b + 1])]
        for h in range(16):
            qv = [bf16(x) for x in qbits[b, h]]
            z = [s * math.fsum(qv[j] * row[j] for j in range(576)) for row in k]
            zm = max(z)
            e = [math.exp(x - zm) for x in z]
            tot = math.fsum(e)
            for d in range(512):
                out[b, h, d] = math.fsum(e[i] * k[i][d] for i in range(len(k))) / tot
    return out


def test_fp8_brute_force_tiny():
    rng = np.random.default_rng(11)
    lens = [1, 3, 2]
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    codes = rng.integers(0, 256, (sum(lens), 576), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A           # no NaN codes
    qbits = _qbits(rng, len(lens))
    kv_scale = 0.0123
    got = dref.mla_decode_ref_fp8(qbits, codes, kv_scale, indptr, SM)
    want = _brute_fp8(qbits, codes, kv_scale, indptr, SM)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-14)


def test_bf16_matches_torch_float64_attention():
    rng = np.random.default_rng(12)
    lens = [5, 17]
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = torch.from_numpy(rng.standard_normal((sum(lens), 576)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    qbits = _qbits(rng, len(lens), 2.0)
    got = dref.mla_decode_ref_bf16(qbits, bits, indptr, SM)
    qf = torch.from_numpy(qbits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    kf = x.to(torch.float64)
    for b in range(len(lens)):
        k = kf[indptr[b]:indptr[b + 1]]
        p = torch.softmax((qf[b] @ k.T) * float(np.float32(SM)), dim=-1)
        np.testing.assert_allclose(got[b], (p @ k[:, :512]).numpy(), rtol=1e-12, atol=1e-15)


def _mxfp4_case(rng, lens, lo=124, hi=128):
    t = sum(lens)
    packed = rng.integers(0, 256, (t, 288), dtype=np.uint8)
    scales = rng.integers(lo, hi + 1, (t, 18), dtype=np.uint8)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return packed, scales, indptr


def test_bf16_cache_of_mxfp4_values_matches_mxfp4_oracle():
    # e2m1 * 2^k is exact in bf16, so the two decoders must agree
    rng = np.random.default_rng(13)
    lens = [4, 33, 1]
    packed, scales, indptr = _mxfp4_case(rng, lens, 110, 140)
    k = mref.dequant_mxfp4(packed, scales)
    bits = torch.from_numpy(k.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(bits.to(torch.float64).numpy(), k)
    bits = bits.view(torch.int16).numpy().view(np.uint16)
    qbits = _qbits(rng, len(lens))
    a = dref.mla_decode_ref_bf16(qbits, bits, indptr, SM)
    b = mref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("kv_scale_log2", [0, -3, 5])
def test_fp8_cache_of_mxfp4_values_matches_mxfp4_oracle(kv_scale_log2):
    # e2m1 * 2^k for k in [-3, 1] is exact in e4m3; a power-of-two per-tensor
    # scale moves the codes without changing the decoded rows
    rng = np.random.default_rng(14 + kv_scale_log2)
    lens = [2, 19]
    packed, scales, indptr = _mxfp4_case(rng, lens)
    k = mref.dequant_mxfp4(packed, scales)
    kv_scale = 2.0 ** kv_scale_log2
    stored = torch.from_numpy(k / kv_scale).to(torch.float8_e4m3fn)
    assert np.array_equal(stored.to(torch.float64).numpy() * kv_scale, k)
    codes = stored.view(torch.uint8).numpy()
    qbits = _qbits(rng, len(lens))
    a = dref.mla_decode_ref_fp8(qbits, codes, kv_scale, indptr, SM)
    b = mref.mla_decode_ref(qbits, packed, scales, indptr, SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_one_token_returns_scaled_v_exactly():
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 0x7E, (1, 576), dtype=np.uint8)
    qbits = _qbits(rng, 1)
    s = 0.37
    out = dref.mla_decode_ref_fp8(qbits, codes, s, [0, 1], SM)
    want = dref.E4M3_VALUES[codes[0, :512]] * np.float64(np.float32(s))
    assert np.array_equal(out[0], np.broadcast_to(want, (16, 512)))
    bits = rng.integers(0, 0x7F00, (1, 576), dtype=np.uint16)
    out = dref.mla_decode_ref_bf16(qbits, bits, [0, 1], SM)
    assert np.array_equal(out[0], np.broadcast_to(mref.bf16_bits_to_f64(bits[0, :512]), (16, 512)))


def test_empty_sequence_gives_zeros():
    rng = np.random.default_rng(16)
    qbits = _qbits(rng, 2)
    codes = rng.integers(0, 0x7E, (3, 576), dtype=np.uint8)
    out = dref.mla_decode_ref_fp8(qbits, codes, 1.0, [0, 0, 3], SM)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


def test_fp8_scale_wiring():
    # out(kv_scale = c, sm) = c * out(kv_scale = 1, c * sm): the per-tensor
    # scale multiplies both the logits and V
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 0x7E, (9, 576), dtype=np.uint8)
    codes[:, ::3] |= 0x80
    qbits = _qbits(rng, 1)
    c = 0.25
    a = dref.mla_decode_ref_fp8(qbits, codes, c, [0, 9], SM)
    b = c * dref.mla_decode_ref_fp8(qbits, codes, 1.0, [0, 9], SM * c)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_permutation_invariance_fp8():
    rng = np.random.default_rng(18)
    codes = rng.integers(0, 0x7E, (40, 576), dtype=np.uint8)
    qbits = _qbits(rng, 1)
    perm = rng.permutation(40)
    a = dref.mla_decode_ref_fp8(qbits, codes, 0.01, [0, 40], SM)
    b = dref.mla_decode_ref_fp8(qbits, codes[perm], 0.01, [0, 40], SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_per_tensor_quantiser():
    # the input generator's fp8 encoding: amax maps to the top code, grid
    # values survive, and every code is the nearest e4m3 value of x / scale
    x = torch.tensor([[3.5, -1.75, 0.0, 0.875, 0.3]], dtype=torch.bfloat16)
    codes, scale = synth.quantize_fp8_per_tensor(x)
    assert float(scale) == np.float32(3.5) / np.float32(448.0)
    # 3.5 -> 448 (0x7E); -1.75 -> -224 = -(1 + 6/8) * 2^7 (0xF6)
    assert int(codes[0, 0]) == 0x7E and int(codes[0, 1]) == 0xF6
    vals = dref.E4M3_VALUES[codes.numpy()]
    y = (x.float() / scale).numpy().astype(np.float64)
    grid = np.unique(dref.E4M3_VALUES[np.isfinite(dref.E4M3_VALUES)])
    for v, t in zip(vals[0], y[0]):
        best = np.min(np.abs(grid - t))
        assert abs(v - t) == best
