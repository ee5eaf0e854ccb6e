"""CPU oracle for MXFP4-KV absorbed-MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it. It shares no code with the HIP library
under ``mla_mxfp4_kv_amd/`` and never imports it.

Sources (kernelindex.com "amd-mixed-mla" leaderboard submission pages):

* page "kernelbot-amd-mixed-mla-608791" -- HIP MXFP4 split-K submission:
  the constants block (16 heads, 576/512 dims, 32-element scale blocks,
  288 packed bytes per token), the ``kFp4Lut`` value table, ``e8m0_to_float``,
  ``unpack_mxfp4`` and the stage-1 tile fill (nibble order, scale index).
* page "kernelbot-amd-mixed-mla-717900" -- Triton MXFP4 flash-decode:
  the layout comment block (nibble order, E8M0 = 2^(byte-127)) and
  ``_nibble_to_f32`` (arithmetic statement of the e2m1 values).
* page "kernelbot-amd-mixed-mla-676098" -- Triton bf16 flash-decode:
  ``_naive_fallback`` (the plain softmax(scale*q.k) v definition with v = the
  first 512 latent dims of the same rows).

Modules:

* :mod:`oracle.mxfp4_ref` -- exact MXFP4 dequantisation and fp64 attention,
  also over per-token row lists (``mla_decode_ref_gather``).
* :mod:`oracle.mxfp4_24_ref` -- the layout with 24 E8M0 bytes per token
  (24-element blocks) from page "kernelbot-amd-mixed-mla-717900".
* :mod:`oracle.dense_ref` -- exact fp8 (e4m3 + per-tensor scale) and bf16
  cache decoding and the same fp64 attention, for the sibling decodes.
* :mod:`oracle.paging_ref` -- page tables (page number, page size, valid rows
  of the last page) expanded to pool rows, page by page.
* :mod:`oracle.planner_ref` -- the CPU reference work-list planner.

Page "kernelbot-amd-mixed-mla-676098" also gives the fp8 cache (``_aiter_mla_decode``:
fp8 rows + one per-tensor scale) and the bf16 cache (``_naive_fallback``).
"""

from .mxfp4_ref import (  # noqa: F401
    E2M1_VALUES,
    NUM_HEADS,
    QK_DIM,
    V_DIM,
    SCALE_BLOCK,
    PACKED_BYTES,
    SCALES_PER_TOKEN,
    bf16_bits_to_f64,
    e2m1_value,
    e8m0_scale,
    dequant_mxfp4,
    mla_decode_ref,
    mla_decode_ref_seq,
    mla_decode_ref_gather,
    mla_decode_ref_page_table,
    mla_decode_ref_groups,
)
from .dense_ref import (  # noqa: F401
    E4M3_VALUES,
    FP8_MAX,
    e4m3_value,
    dequant_fp8,
    dequant_bf16,
    attention_f64,
    mla_decode_ref_fp8,
    mla_decode_ref_fp8_seq,
    mla_decode_ref_bf16,
    mla_decode_ref_bf16_seq,
    mla_decode_ref_fp8_page_table,
    mla_decode_ref_bf16_page_table,
    mla_decode_ref_fp8_groups,
    mla_decode_ref_bf16_groups,
)
from .mxfp4_24_ref import (  # noqa: F401
    SCALE_BLOCK_24,
    SCALES_PER_TOKEN_24,
    dequant_mxfp4_24,
    mla_decode_ref_24,
    mla_decode_ref_24_seq,
)
from .paging_ref import page_table_rows, page_table_token_indptr  # noqa: F401
from .planner_ref import plan_words_ref, PlanRef, decode_plan_words  # noqa: F401
