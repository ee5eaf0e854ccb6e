"""MXFP4 rows with 24 E8M0 scales per token: exact dequantisation and the
fp64 decode over them.

TEST INFRASTRUCTURE ONLY (see the package docstring): a plain CPU statement
of the second MXFP4 scale layout the pages describe. No HIP decode of this
layout exists yet; this module fixes what one must compute.

What differs from :mod:`oracle.mxfp4_ref` (page "kernelbot-amd-mixed-mla-717900",
the mxfp4 layout comment block and the stage-1 tile loads of the Triton
flash-decode):

* A token has 24 E8M0 bytes instead of 18. Scale byte k covers the 24
  consecutive elements ``24k .. 24k+23``, which are the 12 packed bytes
  ``12k .. 12k+11`` of the 288-byte row.
* The packed row is the same: element ``2j`` is the low nibble of byte ``j``,
  element ``2j+1`` the high nibble, each an e2m1 code.
* A scale byte e multiplies by ``2^(e-127)``. Byte 255 is taken as NaN, as
  in the 18-scale layout (page "kernelbot-amd-mixed-mla-608791",
  ``e8m0_to_float``); the Triton page computes the power in fp32 and would
  get +inf there instead, which still makes every non-zero element of the
  block non-finite.
* Attention is unchanged: ``V`` is the first 512 dequantised elements of the
  same row, scores are ``sm_scale * q.K``, softmax over the sequence's
  tokens, zeros for a sequence without tokens (page
  "kernelbot-amd-mixed-mla-676098", ``_naive_fallback``).

The Triton page rounds each dequantised element to bf16 before its dot
products. An e2m1 value times a power of two has at most two significant
bits, so that rounding is exact for every scale byte whose product stays in
bf16's range (bytes 0..254 with |value| below 2^128); the oracle therefore
keeps the exact products in float64.
"""

from __future__ import annotations

import numpy as np

from .dense_ref import attention_f64
from .mxfp4_ref import E2M1_VALUES, NUM_HEADS, PACKED_BYTES, QK_DIM, V_DIM, e8m0_scale

SCALE_BLOCK_24 = 24                          # elements per E8M0 byte
SCALES_PER_TOKEN_24 = QK_DIM // SCALE_BLOCK_24   # 24 bytes per token


def dequant_mxfp4_24(packed, scales) -> np.ndarray:
    """packed: uint8 [T, 288]; scales: uint8 [T, 24] (byte k scales elements
    24k..24k+23). Returns the exact values, float64 [T, 576]."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if packed.ndim != 2 or packed.shape[1] != PACKED_BYTES:
        raise ValueError(f"packed must be [T, {PACKED_BYTES}], got {packed.shape}")
    if scales.shape != (packed.shape[0], SCALES_PER_TOKEN_24):
        raise ValueError(f"scales must be [T, {SCALES_PER_TOKEN_24}], got {scales.shape}")
    codes = np.empty((packed.shape[0], QK_DIM), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return E2M1_VALUES[codes] * np.repeat(e8m0_scale(scales), SCALE_BLOCK_24, axis=1)


def mla_decode_ref_24_seq(q_b, packed_b, scales_b, sm_scale: float) -> np.ndarray:
    """One sequence: float64 [16, 512]."""
    return attention_f64(q_b, dequant_mxfp4_24(packed_b, scales_b), sm_scale)


def mla_decode_ref_24(q, packed, scales, kv_indptr, sm_scale: float, batches=None) -> np.ndarray:
    """The batch over contiguous rows ``kv_indptr[b] .. kv_indptr[b+1]-1``:
    float64 [B, 16, 512] (rows outside ``batches`` are NaN)."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    nb = indptr.shape[0] - 1
    q = np.asarray(q)
    out = np.full((nb, NUM_HEADS, V_DIM), np.nan, dtype=np.float64)
    for b in (range(nb) if batches is None else batches):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        out[b] = mla_decode_ref_24_seq(q[b], packed[lo:hi], scales[lo:hi], sm_scale)
    return out
