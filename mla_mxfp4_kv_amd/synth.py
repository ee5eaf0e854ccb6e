"""Seeded synthetic inputs for MXFP4-KV MLA decode.

This module only MAKES inputs: random bf16 queries, random latent rows and
their MXFP4 encoding (the cache the decode reads). It holds none of the decode
arithmetic (no dequantisation, no attention) and imports neither the HIP
library nor the oracle, so both can be fed from it.

Recipe (one generator, draws in a fixed order: lengths, Q, KV):

* lengths: uniform kv_len, or integers uniform in [lo, hi] inclusive (drawn
  from a CPU generator so the lengths do not depend on the device);
* Q: float32 ``randn * q_std`` rounded to bf16, shape [B, 16, 576];
* KV latent rows: float32 ``randn`` [T, 576], optionally multiplied per token
  by ``2^u`` with u ~ U[-2, 2] (scales log-uniform in [0.25, 4]), rounded to
  bf16, then MXFP4-encoded by :func:`quantize_mxfp4`.

Every draw comes from one CPU ``torch.Generator`` seeded per workload, in
fixed-size row chunks, so a seed always yields the same bytes whatever the
total size and whatever ``device`` is: only the bf16 rows are moved to the
device, where the (exact, integer-valued) MXFP4 encoding runs.

The fp8 and bf16 sibling caches (:func:`make_dense_inputs`) take the same
draws: the bf16 latent rows as they are, or those rows encoded as OCP E4M3
with one per-tensor float32 scale ``amax / 448``, each value divided by it,
clamped to +-448 and rounded to nearest even (the per-tensor recipe page
"kernelbot-amd-mixed-mla-676098" applies to q in ``_aiter_mla_decode``).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

NUM_HEADS = 16
QK_DIM = 576
PACKED_BYTES = 288
SCALES_PER_TOKEN = 18
_ROW_CHUNK = 65536


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    kv_len: int | None          # uniform length, or None when ragged
    ragged: tuple | None        # (lo, hi) inclusive, or None
    q_std: float
    token_scale: bool           # per-token multiplier 2^U[-2,2]
    seed: int
    sm_scale: float = 1.0 / math.sqrt(576.0)


# The five synthetic workloads (shapes of the leaderboard's MI355X decode
# cases plus a long single context and a ragged batch).
WORKLOADS = {
    "b4_kv1024": Workload("b4_kv1024", 4, 1024, None, 1.0, False, 0),
    "b1_kv65536": Workload("b1_kv65536", 1, 65536, None, 1.0, False, 1),
    "b64_kv8192_tokscale": Workload("b64_kv8192_tokscale", 64, 8192, None, 1.0, True, 2),
    "b256_kv8192": Workload("b256_kv8192", 256, 8192, None, 1.0, False, 3),
    "b128_ragged": Workload("b128_ragged", 128, None, (256, 32768), 2.0, False, 4),
}


def quantize_mxfp4(x: torch.Tensor, block: int = 32):
    """MXFP4-encode rows of 576 values (any float dtype, any device).

    Per ``block``-element block (32: 18 scales per token; 24: the 24-scale
    layout of page "kernelbot-amd-mixed-mla-717900"): shared exponent
    ``E = floor(log2(amax)) - 2``
    (exactly, from ``frexp``), stored as the E8M0 byte ``E + 127`` clamped to
    [0, 254]; an all-zero block stores 127. Each element ``x / 2^E`` is rounded
    to the nearest e2m1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the code
    with an even mantissa bit, saturating at 6; the sign bit is set for
    negative inputs. Codes are packed two per byte, element 2j in the low
    nibble of byte j. Returns (packed uint8 [N, 288], scales uint8
    [N, 576 / block]).
    """
    if x.dim() != 2 or x.shape[1] != QK_DIM:
        raise ValueError("x must be [N, 576]")
    if block not in (24, 32):
        raise ValueError("block must be 32 or 24")
    n = x.shape[0]
    xd = x.to(torch.float64).reshape(n, QK_DIM // block, block)
    amax = xd.abs().amax(dim=2)
    _, e = torch.frexp(amax)                     # amax = m * 2^e, m in [0.5, 1)
    byte = (e.to(torch.int32) - 3 + 127).clamp(0, 254)
    byte = torch.where(amax > 0, byte, torch.full_like(byte, 127))
    shift = (byte - 127).to(torch.float64)
    y = xd * torch.exp2(-shift).unsqueeze(2)     # exact: power-of-two scaling in fp64
    a = y.abs()
    # Rounding thresholds between consecutive magnitude codes; at a tie the
    # even code wins, so the comparison is strict before an odd code and
    # inclusive before an even one.
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8)
            + (a > 1.25).to(torch.uint8) + (a >= 1.75).to(torch.uint8)
            + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
            + (a > 5.0).to(torch.uint8))
    code = code | ((y < 0).to(torch.uint8) << 3)
    code = code.reshape(n, QK_DIM)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, byte.to(torch.uint8).contiguous()


def seq_lengths(w: Workload) -> list:
    """Per-sequence KV lengths of a workload (device independent)."""
    if w.ragged is None:
        return [int(w.kv_len)] * w.batch
    g = torch.Generator().manual_seed(w.seed)
    lo, hi = w.ragged
    return [int(v) for v in torch.randint(lo, hi + 1, (w.batch,), generator=g)]


def _draw(w: Workload, device, lengths):
    """Lengths, bf16 Q and a generator of (row0, row1, bf16 latent rows)
    chunks, in the fixed draw order."""
    device = torch.device(device)
    lens = seq_lengths(w) if lengths is None else [int(v) for v in lengths]
    batch = len(lens)
    indptr = [0]
    for n in lens:
        indptr.append(indptr[-1] + n)
    total = indptr[-1]
    g = torch.Generator().manual_seed(w.seed + 1000)   # CPU: the bytes do not depend on `device`
    q = (torch.randn(batch, NUM_HEADS, QK_DIM, generator=g, dtype=torch.float32)
         * w.q_std).to(torch.bfloat16).to(device)

    def rows():
        for r0 in range(0, total, _ROW_CHUNK):
            r1 = min(total, r0 + _ROW_CHUNK)
            x = torch.randn(r1 - r0, QK_DIM, generator=g, dtype=torch.float32)
            if w.token_scale:
                u = torch.rand(r1 - r0, 1, generator=g, dtype=torch.float32)
                x = x * torch.exp2(4.0 * u - 2.0)
            yield r0, r1, x.to(torch.bfloat16).to(device)

    return lens, torch.tensor(indptr, dtype=torch.int32), total, q, rows()


def make_inputs(w: Workload, device="cpu", lengths=None, block: int = 32):
    """Build (q bf16 [B,16,576], packed u8 [T,288], scales u8 [T,576/block],
    kv_indptr int32 [B+1] on the host, lengths list) on ``device``.

    ``lengths`` overrides the workload's length rule (for small test cases);
    ``block`` 24 gives the 24-scale cache of the same draws.
    """
    lens, kv_indptr, total, q, rows = _draw(w, device, lengths)
    packed = torch.empty(total, PACKED_BYTES, dtype=torch.uint8, device=q.device)
    scales = torch.empty(total, QK_DIM // block, dtype=torch.uint8, device=q.device)
    for r0, r1, x in rows:
        pk, sc = quantize_mxfp4(x, block)
        packed[r0:r1] = pk
        scales[r0:r1] = sc
    return q, packed, scales, kv_indptr, lens


FP8_MAX = 448.0


def quantize_fp8_per_tensor(x: torch.Tensor):
    """OCP E4M3 codes (uint8, same shape) of ``x`` and the per-tensor float32
    scale (a 1-element tensor): scale = amax / 448 (1 for an all-zero
    tensor), codes = e4m3(clamp(x / scale, -448, 448)) rounded to nearest
    even."""
    amax = x.abs().amax().to(torch.float32) if x.numel() else torch.zeros((), device=x.device)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).reshape(1)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    flat = x.reshape(-1, x.shape[-1]) if x.dim() > 1 else x.reshape(1, -1)
    out = codes.view(flat.shape)
    for r0 in range(0, flat.shape[0], _ROW_CHUNK):
        y = (flat[r0:r0 + _ROW_CHUNK].to(torch.float32) / scale).clamp(-FP8_MAX, FP8_MAX)
        out[r0:r0 + _ROW_CHUNK] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_dense_inputs(w: Workload, fmt: str, device="cpu", lengths=None):
    """The sibling caches of a workload, from the same draws as
    :func:`make_inputs`: returns (q bf16 [B,16,576], cache, kv_scale,
    kv_indptr int32 [B+1] on the host, lengths) with
    * fmt "bf16": cache = the bf16 latent rows [T, 576], kv_scale None;
    * fmt "fp8": cache = uint8 E4M3 codes [T, 576], kv_scale float32 [1].
    """
    if fmt not in ("bf16", "fp8"):
        raise ValueError(f"unknown cache format {fmt!r}")
    lens, kv_indptr, total, q, rows = _draw(w, device, lengths)
    lat = torch.empty(total, QK_DIM, dtype=torch.bfloat16, device=q.device)
    for r0, r1, x in rows:
        lat[r0:r1] = x
    if fmt == "bf16":
        return q, lat, None, kv_indptr, lens
    codes, scale = quantize_fp8_per_tensor(lat)
    del lat
    return q, codes, scale, kv_indptr, lens


KV_BYTES_PER_TOKEN = {"mxfp4": PACKED_BYTES + SCALES_PER_TOKEN, "mxfp4_24": PACKED_BYTES + 24, "fp8": QK_DIM,
                      "bf16": 2 * QK_DIM}


def kv_bytes(total_tokens: int, fmt: str = "mxfp4") -> int:
    """Algorithmic KV-cache bytes a decode call must read: packed rows +
    E8M0 scales (mxfp4, 306 B/token; mxfp4_24, 312 B/token), fp8 rows (576 B/token; the one
    per-tensor scale is negligible) or bf16 rows (1152 B/token)."""
    return total_tokens * KV_BYTES_PER_TOKEN[fmt]
