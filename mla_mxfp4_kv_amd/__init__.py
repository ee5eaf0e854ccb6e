"""MXFP4-KV absorbed-MLA decode for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI shared library built from ``csrc/``
(``libmla_mxfp4.so``); :mod:`mla_mxfp4_kv_amd.binding` is a thin ctypes layer
over it that only marshals pointers and sizes. :mod:`mla_mxfp4_kv_amd.synth`
builds seeded synthetic inputs.
"""
