"""Exact MXFP4 dequantisation and fp64 absorbed-MLA decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): a plain, slow CPU
statement of what the decode computes, used to check the HIP library.

What is computed, for every sequence b and head h (q_seq_len = 1):

1. The tokens of sequence b are rows ``kv_indptr[b] .. kv_indptr[b+1]-1`` of
   the packed cache ("kernelbot-amd-mixed-mla-608791", stage-1 kernel: the
   work range is a slice of the contiguous token rows; page size 1).
2. Element j (0..575) of token t sits in byte ``j // 2`` of the token's
   288-byte row: low nibble for even j, high nibble for odd j
   ("kernelbot-amd-mixed-mla-608791", tile fill in the stage-1 kernel;
   "kernelbot-amd-mixed-mla-717900", the mxfp4 layout comment block).
3. The nibble is an OCP e2m1 code; its value is the ``kFp4Lut`` table
   ("kernelbot-amd-mixed-mla-608791", constants block).
4. The element is multiplied by the E8M0 block scale ``2^(byte-127)`` of block
   ``j // 32`` (18 blocks per token); byte 255 is NaN and byte 0 is 2^-127
   ("kernelbot-amd-mixed-mla-608791", ``e8m0_to_float``; the 717900 page's
   layout comment gives the same power-of-two rule).
5. ``K[t, :]`` is the 576-wide dequantised row and ``V[t, :] = K[t, :512]``;
   scores ``z_t = sm_scale * sum_j q[b,h,j] K[t,j]``; ``p = softmax(z)``;
   ``out[b,h,:] = sum_t p_t V[t,:]`` ("kernelbot-amd-mixed-mla-676098",
   ``_naive_fallback``). No mask, no logit cap.
6. A sequence with no tokens produces zeros ("kernelbot-amd-mixed-mla-608791",
   reduce kernel: all-empty splits write zeros).

Everything is evaluated in float64. Each product bf16 x (e2m1 * 2^k) is exact
in fp64, so the only rounding is in the fp64 sums and exp.
"""

from __future__ import annotations

import numpy as np

# Shapes fixed by the constants block of "kernelbot-amd-mixed-mla-608791".
NUM_HEADS = 16
QK_DIM = 576          # 512 latent + 64 rope
V_DIM = 512           # V = first 512 latent dims
SCALE_BLOCK = 32      # elements per E8M0 scale
PACKED_BYTES = QK_DIM // 2            # 288 bytes of fp4x2 per token
SCALES_PER_TOKEN = QK_DIM // SCALE_BLOCK  # 18 E8M0 bytes per token

# The e2m1 value table, code 0..15 ("kernelbot-amd-mixed-mla-608791",
# ``kFp4Lut``). Code 8 is negative zero.
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
    dtype=np.float64,
)


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code, from the ``kFp4Lut`` table."""
    return float(E2M1_VALUES[int(code) & 0xF])


def e8m0_scale(byte) -> np.ndarray:
    """E8M0 scale byte -> float64 multiplier ``2^(byte-127)``; 255 -> NaN.

    ("kernelbot-amd-mixed-mla-608791", ``e8m0_to_float``: byte 0 is the
    smallest power 2^-127, byte 255 is a NaN pattern.)
    """
    e = np.asarray(byte, dtype=np.int64)
    out = np.ldexp(1.0, e - 127).astype(np.float64)
    return np.where(e == 255, np.nan, out)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_mxfp4(packed, scales) -> np.ndarray:
    """Exact dequantisation of MXFP4 rows.

    packed: uint8 [T, 288] (two e2m1 codes per byte, low nibble first);
    scales: uint8 [T, 18] (E8M0, one per 32 consecutive elements).
    Returns float64 [T, 576].
    """
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if packed.ndim != 2 or packed.shape[1] != PACKED_BYTES:
        raise ValueError(f"packed must be [T, {PACKED_BYTES}], got {packed.shape}")
    if scales.shape != (packed.shape[0], SCALES_PER_TOKEN):
        raise ValueError(f"scales must be [T, {SCALES_PER_TOKEN}], got {scales.shape}")
    t = packed.shape[0]
    codes = np.empty((t, QK_DIM), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F     # element 2j: low nibble of byte j
    codes[:, 1::2] = packed >> 4       # element 2j+1: high nibble of byte j
    values = E2M1_VALUES[codes]
    block_scale = e8m0_scale(scales)   # [T, 18]
    return values * np.repeat(block_scale, SCALE_BLOCK, axis=1)


def _as_q_f64(q) -> np.ndarray:
    q = np.asarray(q)
    if q.dtype == np.uint16:
        return bf16_bits_to_f64(q)
    return q.astype(np.float64)


def mla_decode_ref_seq(q_b, packed_b, scales_b, sm_scale: float) -> np.ndarray:
    """Attention output of one sequence: float64 [16, 512].

    q_b: [16, 576] (bf16 bit patterns as uint16, or exact float values);
    packed_b / scales_b: that sequence's rows of the cache.
    """
    qf = _as_q_f64(q_b)
    if qf.shape != (NUM_HEADS, QK_DIM):
        raise ValueError(f"q row must be [{NUM_HEADS}, {QK_DIM}], got {qf.shape}")
    n = np.asarray(packed_b).shape[0]
    if n == 0:
        return np.zeros((NUM_HEADS, V_DIM), dtype=np.float64)
    k = dequant_mxfp4(packed_b, scales_b)           # [n, 576]
    v = k[:, :V_DIM]                                 # [n, 512]
    s = np.float64(np.float32(sm_scale))
    z = s * (qf @ k.T)                               # [16, n]
    zmax = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - zmax)
    p = e / np.sum(e, axis=1, keepdims=True)
    return p @ v


def mla_decode_ref(q, packed, scales, kv_indptr, sm_scale: float,
                   batches=None) -> np.ndarray:
    """Oracle for the whole batch: float64 [B, 16, 512].

    q: [B, 16, 576]; packed: uint8 [T, 288]; scales: uint8 [T, 18];
    kv_indptr: int [B+1] prefix offsets into the token rows.
    ``batches`` optionally restricts the work to some sequences (the other
    rows of the result are left as NaN).
    """
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    nb = indptr.shape[0] - 1
    q = np.asarray(q)
    out = np.full((nb, NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    todo = range(nb) if batches is None else batches
    for b in todo:
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        out[b] = mla_decode_ref_seq(q[b], packed[lo:hi], scales[lo:hi], sm_scale)
    return out


def mla_decode_ref_gather(q, packed, scales, kv_indices, kv_indptr, sm_scale: float,
                          batches=None) -> np.ndarray:
    """Oracle for a cache whose token rows are listed per token: sequence b
    reads rows ``kv_indices[kv_indptr[b] : kv_indptr[b+1]]`` of the row pool
    (page size 1, the layout the decode call on page
    "kernelbot-amd-mixed-mla-676098" describes with ``kv_indices`` and
    ``page_size=1``). Otherwise the same definition: float64 [B, 16, 512]."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    idx = np.asarray(kv_indices, dtype=np.int64)
    nb = indptr.shape[0] - 1
    q = np.asarray(q)
    out = np.full((nb, NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for b in (range(nb) if batches is None else batches):
        rows = idx[int(indptr[b]):int(indptr[b + 1])]
        out[b] = mla_decode_ref_seq(q[b], np.asarray(packed)[rows], np.asarray(scales)[rows], sm_scale)
    return out


def mla_decode_ref_page_table(q, packed, scales, page_indices, page_indptr, kv_last_page_len,
                              page_size: int, sm_scale: float, batches=None) -> np.ndarray:
    """Oracle over a page table (``oracle.paging_ref``): each sequence's pool
    rows, page by page, then the same definition. float64 [B, 16, 512]."""
    from .paging_ref import page_table_rows
    rows = page_table_rows(page_indices, page_indptr, kv_last_page_len, page_size)
    q = np.asarray(q)
    out = np.full((len(rows), NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for b in (range(len(rows)) if batches is None else batches):
        out[b] = mla_decode_ref_seq(q[b], np.asarray(packed)[rows[b]], np.asarray(scales)[rows[b]], sm_scale)
    return out


def mla_decode_ref_groups(q, packed, scales, kv_indptr, groups: int, sm_scale: float,
                          batches=None) -> np.ndarray:
    """Query entries sharing their sequence's rows: entry e holds the 16
    heads of query group e % groups of sequence e // groups (page
    "kernelbot-amd-mixed-mla-676098": the Triton decode maps query token i
    to sequence i // q_seq_len; a 128-head query is 8 such groups) and
    attends all of that sequence's rows. float64 [E, 16, 512]."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    q = np.asarray(q)
    out = np.full((q.shape[0], NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for e in (range(q.shape[0]) if batches is None else batches):
        b = e // groups
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        out[e] = mla_decode_ref_seq(q[e], np.asarray(packed)[lo:hi], np.asarray(scales)[lo:hi], sm_scale)
    return out
