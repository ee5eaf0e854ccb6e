"""Exact fp8 (e4m3) and bf16 KV-cache decoding and fp64 absorbed-MLA decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): a plain, slow CPU
statement of what the fp8-KV and bf16-KV sibling decodes compute, used to
check the HIP library.

The attention is the same definition as for the MXFP4 cache (page
"kernelbot-amd-mixed-mla-676098", ``_naive_fallback``): for every sequence b
and head h, ``out[b,h,:] = sum_t softmax_t(sm_scale * q[b,h,:] . K[t,:]) V[t,:]``
with ``V[t,:] = K[t,:512]``. Only the cache format differs:

* bf16 cache: ``K[t,:]`` is row t of a bfloat16 [T, 576] tensor (page
  "kernelbot-amd-mixed-mla-676098", ``_naive_fallback`` reads
  ``kv_data["bf16"]`` rows of 576 values and widens them to float).
* fp8 cache: row t of an fp8 [T, 576] tensor times one per-tensor float32
  scale (page "kernelbot-amd-mixed-mla-676098", ``_aiter_mla_decode``:
  ``kv_fp8, kv_scale = kv_data["fp8"]``, the scale handed to the decode with
  the fp8 rows). The fp8 type is the one the page takes from the tensor's
  dtype; on MI355X that is OCP FP8 E4M3 ("e4m3fn", largest finite value
  448, the ``finfo.max`` the pages clamp to; page
  "kernelbot-amd-mixed-mla-717900", constants ``FP8_MAX``/``FP8_MIN``).

E4M3 codes (OCP 8-bit floating point, E4M3 variant): sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
``m/8 * 2^-6``; the codes with all exponent and mantissa bits set (0x7F,
0xFF) are NaN; there are no infinities.

Everything is evaluated in float64. An e4m3 value (4 significant bits) times
the float32 scale (24 bits), or a bf16 value (8 bits), is exact in fp64, and
so is its product with a bf16 query element (at most 36 bits); the only
rounding is in the fp64 sums and exp.
"""

from __future__ import annotations

import numpy as np

from .mxfp4_ref import NUM_HEADS, QK_DIM, V_DIM, bf16_bits_to_f64

FP8_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (0..255) from its bit fields."""
    code = int(code) & 0xFF
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


# Value of every code, by index.
E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequant_fp8(codes, kv_scale) -> np.ndarray:
    """fp8 rows (uint8 codes [T, 576]) times the per-tensor float32 scale,
    exactly, as float64 [T, 576]."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.ndim != 2 or codes.shape[1] != QK_DIM:
        raise ValueError(f"fp8 rows must be [T, {QK_DIM}], got {codes.shape}")
    s = np.float64(np.float32(kv_scale))
    return E4M3_VALUES[codes] * s


def dequant_bf16(bits) -> np.ndarray:
    """bf16 rows (uint16 bit patterns [T, 576]) as exact float64 [T, 576]."""
    bits = np.asarray(bits)
    if bits.ndim != 2 or bits.shape[1] != QK_DIM:
        raise ValueError(f"bf16 rows must be [T, {QK_DIM}], got {bits.shape}")
    return bf16_bits_to_f64(bits)


def attention_f64(q_b, k, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q K^T) V for one sequence in float64: q_b [16, 576]
    (bf16 bits as uint16, or float values), k float64 [n, 576]; V = k[:, :512].
    No tokens -> zeros (the reduce kernel of page
    "kernelbot-amd-mixed-mla-608791" writes zeros for an all-empty split)."""
    q_b = np.asarray(q_b)
    qf = bf16_bits_to_f64(q_b) if q_b.dtype == np.uint16 else q_b.astype(np.float64)
    if qf.shape != (NUM_HEADS, QK_DIM):
        raise ValueError(f"q row must be [{NUM_HEADS}, {QK_DIM}], got {qf.shape}")
    if k.shape[0] == 0:
        return np.zeros((NUM_HEADS, V_DIM), dtype=np.float64)
    s = np.float64(np.float32(sm_scale))
    z = s * (qf @ k.T)                                # [16, n]
    zmax = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - zmax)
    p = e / np.sum(e, axis=1, keepdims=True)
    return p @ k[:, :V_DIM]


def mla_decode_ref_fp8_seq(q_b, codes_b, kv_scale, sm_scale: float) -> np.ndarray:
    """One sequence over an fp8 cache: float64 [16, 512]."""
    return attention_f64(q_b, dequant_fp8(codes_b, kv_scale), sm_scale)


def mla_decode_ref_bf16_seq(q_b, bits_b, sm_scale: float) -> np.ndarray:
    """One sequence over a bf16 cache: float64 [16, 512]."""
    return attention_f64(q_b, dequant_bf16(bits_b), sm_scale)


def _batched(fn, q, kv_indptr, batches):
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    nb = indptr.shape[0] - 1
    out = np.full((nb, NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for b in (range(nb) if batches is None else batches):
        out[b] = fn(np.asarray(q)[b], int(indptr[b]), int(indptr[b + 1]))
    return out


def mla_decode_ref_fp8(q, codes, kv_scale, kv_indptr, sm_scale: float, batches=None):
    """Oracle for a batch over an fp8 cache: float64 [B, 16, 512] (rows not
    in ``batches`` are left NaN)."""
    return _batched(lambda qb, lo, hi: mla_decode_ref_fp8_seq(qb, codes[lo:hi], kv_scale, sm_scale),
                    q, kv_indptr, batches)


def mla_decode_ref_bf16(q, bits, kv_indptr, sm_scale: float, batches=None):
    """Oracle for a batch over a bf16 cache: float64 [B, 16, 512]."""
    return _batched(lambda qb, lo, hi: mla_decode_ref_bf16_seq(qb, bits[lo:hi], sm_scale),
                    q, kv_indptr, batches)


def _page_table(fn, q, page_indices, page_indptr, kv_last_page_len, page_size, batches):
    from .paging_ref import page_table_rows
    rows = page_table_rows(page_indices, page_indptr, kv_last_page_len, page_size)
    out = np.full((len(rows), NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for b in (range(len(rows)) if batches is None else batches):
        out[b] = fn(np.asarray(q)[b], rows[b])
    return out


def mla_decode_ref_fp8_page_table(q, codes, kv_scale, page_indices, page_indptr, kv_last_page_len,
                                  page_size: int, sm_scale: float, batches=None):
    """fp8 oracle over a page table (``oracle.paging_ref``): float64 [B, 16, 512]."""
    return _page_table(lambda qb, r: mla_decode_ref_fp8_seq(qb, np.asarray(codes)[r], kv_scale, sm_scale),
                       q, page_indices, page_indptr, kv_last_page_len, page_size, batches)


def mla_decode_ref_bf16_page_table(q, bits, page_indices, page_indptr, kv_last_page_len, page_size: int,
                                   sm_scale: float, batches=None):
    """bf16 oracle over a page table: float64 [B, 16, 512]."""
    return _page_table(lambda qb, r: mla_decode_ref_bf16_seq(qb, np.asarray(bits)[r], sm_scale),
                       q, page_indices, page_indptr, kv_last_page_len, page_size, batches)


def _groups(fn, q, kv_indptr, groups, batches):
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    q = np.asarray(q)
    out = np.full((q.shape[0], NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for e in (range(q.shape[0]) if batches is None else batches):
        b = e // groups
        out[e] = fn(q[e], int(indptr[b]), int(indptr[b + 1]))
    return out


def mla_decode_ref_fp8_groups(q, codes, kv_scale, kv_indptr, groups: int, sm_scale: float, batches=None):
    """fp8 oracle for query entries sharing their sequence's rows (entry e
    reads sequence e // groups): float64 [E, 16, 512]."""
    return _groups(lambda qb, lo, hi: mla_decode_ref_fp8_seq(qb, codes[lo:hi], kv_scale, sm_scale),
                   q, kv_indptr, groups, batches)


def mla_decode_ref_bf16_groups(q, bits, kv_indptr, groups: int, sm_scale: float, batches=None):
    """bf16 oracle for query entries sharing their sequence's rows."""
    return _groups(lambda qb, lo, hi: mla_decode_ref_bf16_seq(qb, bits[lo:hi], sm_scale),
                   q, kv_indptr, groups, batches)
