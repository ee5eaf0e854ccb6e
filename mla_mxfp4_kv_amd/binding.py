"""ctypes binding of libmla_mxfp4.so (argument marshalling only).

Every function here forwards plain pointers and sizes to the C ABI declared in
``include/mla_mxfp4.h``; all computation happens in the library's HIP
kernels. PyTorch is used only for device memory and the current stream. If the
library is missing this module raises on first use -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_mxfp4.so")

MLA_OK = 0
NUM_HEADS = 16
QK_DIM = 576
V_DIM = 512
PACKED_BYTES = 288
SCALES_PER_TOKEN = 18

# Every symbol the header declares (checked by the CPU test suite).
EXPORTS = (
    "mla_status_string", "mla_last_error", "mla_device_num_cus", "mla_workspace_bytes",
    "mla_plan", "mla_plan_cus", "mla_plan_device", "mla_plan_release", "mla_plan_host", "mla_decode_mxfp4",
    "mla_decode_fp8", "mla_decode_bf16", "mla_decode_mxfp4_paged", "mla_decode_fp8_paged",
    "mla_decode_bf16_paged", "mla_decode_mxfp4_page_table", "mla_decode_fp8_page_table",
    "mla_decode_bf16_page_table", "mla_decode_mxfp4_starts", "mla_decode_fp8_starts", "mla_decode_bf16_starts",
    "mla_decode_mxfp4_noalloc", "mla_decode_mxfp4_24",
)

_lib = None


class MlaError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with {status}: {msg}")
        self.status = status


def lib():
    """Load the shared library once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_mxfp4_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_i32p = ctypes.POINTER(ctypes.c_int32)
    c_sizep = ctypes.POINTER(ctypes.c_size_t)
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_device_num_cus.argtypes = [c_i32p]
    L.mla_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, c_sizep]
    L.mla_plan.argtypes = [c_i32p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.mla_plan_cus.argtypes = [c_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]
    L.mla_plan_device.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.mla_plan_host.argtypes = [c_i32p, ctypes.c_int32, ctypes.c_int32, c_i32p, ctypes.c_size_t,
                                c_sizep, c_sizep]
    L.mla_plan_release.argtypes = [ctypes.c_void_p]
    L.mla_decode_mxfp4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_mxfp4_24.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_mxfp4_noalloc.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                                                                   ctypes.c_void_p]
    L.mla_decode_mxfp4_paged.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                         ctypes.c_void_p]
    L.mla_decode_fp8_paged.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_bf16_paged.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    # (q, pool, [scale,] page_indices, page_indptr, page_size, kv_indptr, out, sm_scale, workspace, stream)
    pt = [ctypes.c_void_p] * 5 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                   ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_mxfp4_page_table.argtypes = pt
    L.mla_decode_fp8_page_table.argtypes = pt
    L.mla_decode_bf16_page_table.argtypes = pt[:1] + pt[2:]
    # (q, pool, [scale,] kv_start, kv_indptr, out, sm_scale, workspace, stream)
    st = [ctypes.c_void_p] * 6 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_mxfp4_starts.argtypes = st
    L.mla_decode_fp8_starts.argtypes = st
    L.mla_decode_bf16_starts.argtypes = st[:1] + st[2:]
    for name in ("mla_device_num_cus", "mla_workspace_bytes", "mla_plan", "mla_plan_cus",
                 "mla_plan_device", "mla_plan_release", "mla_plan_host", "mla_decode_mxfp4", "mla_decode_fp8",
                 "mla_decode_bf16", "mla_decode_mxfp4_paged", "mla_decode_fp8_paged",
                 "mla_decode_bf16_paged", "mla_decode_mxfp4_page_table", "mla_decode_fp8_page_table",
                 "mla_decode_bf16_page_table", "mla_decode_mxfp4_starts", "mla_decode_fp8_starts",
                 "mla_decode_bf16_starts", "mla_decode_mxfp4_noalloc", "mla_decode_mxfp4_24"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, fn: str):
    if status != MLA_OK:
        msg = lib().mla_last_error().decode(errors="replace")
        raise MlaError(status, fn, msg)


def _indptr_array(kv_indptr):
    vals = [int(v) for v in kv_indptr]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals), len(vals) - 1


def status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def num_cus() -> int:
    n = ctypes.c_int32(0)
    _check(lib().mla_device_num_cus(ctypes.byref(n)), "mla_device_num_cus")
    return n.value


_device_num_cus = num_cus   # for callers whose own argument is named num_cus


def workspace_bytes(batch: int, total_kv: int, num_cus: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().mla_workspace_bytes(batch, total_kv, num_cus, ctypes.byref(out)),
           "mla_workspace_bytes")
    return out.value


def plan_host(kv_indptr, num_cus: int):
    """Host planner words for ``kv_indptr`` (list of B+1 ints) -> (words, bytes)."""
    arr, batch = _indptr_array(kv_indptr)
    n = ctypes.c_size_t(0)
    need = ctypes.c_size_t(0)
    st = lib().mla_plan_host(arr, batch, num_cus, None, 0, ctypes.byref(n), ctypes.byref(need))
    if st not in (MLA_OK, -2):
        _check(st, "mla_plan_host")
    words = (ctypes.c_int32 * max(1, n.value))()
    _check(lib().mla_plan_host(arr, batch, num_cus, words, n.value, ctypes.byref(n),
                               ctypes.byref(need)), "mla_plan_host")
    return list(words[: n.value]), need.value


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def plan(kv_indptr_host, workspace, num_cus: int = 0, stream=None):
    """Build the work list for ``kv_indptr_host`` into the device tensor
    ``workspace`` (uint8, 256-byte aligned)."""
    arr, batch = _indptr_array(kv_indptr_host)
    _check(lib().mla_plan_cus(arr, batch, num_cus, ctypes.c_void_p(workspace.data_ptr()),
                              workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "mla_plan")


def plan_device(kv_indptr_dev, batch: int, max_total_kv: int, workspace, num_cus: int = 0,
                stream=None):
    """Enqueue the GPU-side planner for the device tensor ``kv_indptr_dev``
    (int32 [batch+1]) into ``workspace`` (no host synchronisation)."""
    _check(lib().mla_plan_device(ctypes.c_void_p(kv_indptr_dev.data_ptr()), batch, max_total_kv,
                                 num_cus, ctypes.c_void_p(workspace.data_ptr()),
                                 workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "mla_plan_device")


def plan_release(workspace_ptr: int) -> int:
    """Forget the plan registered for a workspace address (host record only);
    returns the status (MLA_OK, or -5 when nothing was registered)."""
    return lib().mla_plan_release(ctypes.c_void_p(workspace_ptr))


def _release_on_free(workspace):
    """Release the workspace's plan record when the tensor is collected, so a
    later tensor at the same address is refused until it is planned."""
    import weakref
    fin = weakref.finalize(workspace, plan_release, workspace.data_ptr())
    fin.atexit = False


def decode(q, kv_packed, kv_scale, kv_indptr_dev, out, sm_scale: float, workspace, stream=None):
    """Enqueue the decode of a planned workspace on ``stream`` (no sync)."""
    _check(lib().mla_decode_mxfp4(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_packed.data_ptr()),
        ctypes.c_void_p(kv_scale.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale),
        ctypes.c_void_p(workspace.data_ptr()), _stream_ptr(stream)), "mla_decode_mxfp4")


def decode_noalloc(q, kv_packed, kv_scale, kv_indptr_dev, batch: int, out, sm_scale: float, stream=None):
    """Enqueue the decode that allocates nothing (plan and partials in the
    library's static device array; the plan is built on the GPU from the
    device offsets). Calls on one GPU share that array: order them."""
    _check(lib().mla_decode_mxfp4_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_packed.data_ptr()),
        ctypes.c_void_p(kv_scale.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()), batch,
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale), _stream_ptr(stream)), "mla_decode_mxfp4_noalloc")


def decode_mxfp4_paged(q, kv_packed, kv_scale, kv_indices, kv_indptr_dev, out, sm_scale: float, workspace,
                       stream=None):
    """Enqueue the MXFP4 decode over per-token row lists (no checks; see
    ``MlaDecode.mxfp4_paged``)."""
    _check(lib().mla_decode_mxfp4_paged(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_packed.data_ptr()),
        ctypes.c_void_p(kv_scale.data_ptr()), ctypes.c_void_p(kv_indices.data_ptr()),
        ctypes.c_void_p(kv_indptr_dev.data_ptr()), ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale),
        ctypes.c_void_p(workspace.data_ptr()), _stream_ptr(stream)), "mla_decode_mxfp4_paged")


def decode_fp8_paged(q, kv_fp8, kv_scale, kv_indices, kv_indptr_dev, out, sm_scale: float, workspace,
                     stream=None):
    """Enqueue the fp8 decode over per-token row lists (no checks)."""
    _check(lib().mla_decode_fp8_paged(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_fp8.data_ptr()), ctypes.c_void_p(kv_scale.data_ptr()),
        ctypes.c_void_p(kv_indices.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale), ctypes.c_void_p(workspace.data_ptr()),
        _stream_ptr(stream)), "mla_decode_fp8_paged")


def decode_bf16_paged(q, kv_bf16, kv_indices, kv_indptr_dev, out, sm_scale: float, workspace, stream=None):
    """Enqueue the bf16 decode over per-token row lists (no checks)."""
    _check(lib().mla_decode_bf16_paged(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_bf16.data_ptr()),
        ctypes.c_void_p(kv_indices.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale), ctypes.c_void_p(workspace.data_ptr()),
        _stream_ptr(stream)), "mla_decode_bf16_paged")


def check_kv_indices(kv_indices, kv_indptr_host, pool_rows: int, row_bytes: int = PACKED_BYTES):
    """Host-side guard for gathered caches: int32 contiguous device indices
    covering kv_indptr[-1] tokens, all in [0, pool_rows) (reads the indices
    back, one synchronisation), and a pool small enough for 32-bit offsets."""
    import torch
    if kv_indices.dtype != torch.int32 or kv_indices.dim() != 1 or not kv_indices.is_contiguous():
        raise ValueError("kv_indices must be a contiguous int32 tensor")
    hi_tok = int(kv_indptr_host[-1]) if len(kv_indptr_host) else 0
    lo_tok = int(kv_indptr_host[0]) if len(kv_indptr_host) else 0
    if kv_indices.numel() < hi_tok:
        raise ValueError("kv_indices is shorter than kv_indptr[-1]")
    if pool_rows * row_bytes >= 2 ** 32:
        raise ValueError("the row pool must be smaller than 2^32 bytes")
    if hi_tok > lo_tok:
        used = kv_indices[lo_tok:hi_tok]
        if int(used.min()) < 0 or int(used.max()) >= pool_rows:
            raise ValueError("kv_indices holds rows outside the pool")


def decode_page_table(fmt: str, q, pool, kv_scale, page_indices, page_indptr_dev, page_size: int, kv_indptr_dev,
                      out, sm_scale: float, workspace, stream=None):
    """Enqueue a decode over a page table (no checks; see ``MlaDecodePageTable``).
    ``fmt``: "mxfp4" (pool = packed rows, kv_scale = E8M0 rows), "fp8" (kv_scale
    = float32 [1]) or "bf16" (kv_scale unused)."""
    head = [ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(pool.data_ptr())]
    if fmt != "bf16":
        head.append(ctypes.c_void_p(kv_scale.data_ptr()))
    fn = f"mla_decode_{fmt}_page_table"
    _check(getattr(lib(), fn)(
        *head, ctypes.c_void_p(page_indices.data_ptr()), ctypes.c_void_p(page_indptr_dev.data_ptr()),
        ctypes.c_int32(page_size), ctypes.c_void_p(kv_indptr_dev.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_float(sm_scale), ctypes.c_void_p(workspace.data_ptr()), _stream_ptr(stream)), fn)


def decode_starts(fmt: str, q, pool, kv_scale, kv_start_dev, kv_indptr_dev, out, sm_scale: float, workspace,
                  stream=None):
    """Enqueue a decode over shared contiguous rows (no checks; see ``MlaDecodeGroups``)."""
    head = [ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(pool.data_ptr())]
    if fmt != "bf16":
        head.append(ctypes.c_void_p(kv_scale.data_ptr()))
    fn = f"mla_decode_{fmt}_starts"
    _check(getattr(lib(), fn)(
        *head, ctypes.c_void_p(kv_start_dev.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale), ctypes.c_void_p(workspace.data_ptr()),
        _stream_ptr(stream)), fn)


def page_table_kv_indptr(page_indptr, kv_last_page_len, page_size: int):
    """Token offsets of a page table: sequence b holds (pages - 1) * page_size
    + kv_last_page_len[b] tokens (none without pages). Checks that the page
    offsets are non-decreasing from >= 0 and that every non-empty sequence's
    last page holds 1..page_size rows."""
    pi = [int(v) for v in page_indptr]
    last = [int(v) for v in kv_last_page_len]
    if page_size < 1:
        raise ValueError("page_size must be >= 1")
    if len(pi) < 1 or len(last) != len(pi) - 1:
        raise ValueError("page_indptr needs batch + 1 entries and kv_last_page_len batch entries")
    if pi[0] < 0 or any(b < a for a, b in zip(pi, pi[1:])):
        raise ValueError("page_indptr must be non-decreasing from a value >= 0")
    tok = [0]
    for b in range(len(last)):
        n = pi[b + 1] - pi[b]
        if n > 0 and not 1 <= last[b] <= page_size:
            raise ValueError(f"kv_last_page_len[{b}] = {last[b]} is not in [1, page_size]")
        tok.append(tok[-1] + ((n - 1) * page_size + last[b] if n > 0 else 0))
    if tok[-1] >= 2 ** 31:
        raise ValueError("more than 2^31 - 1 tokens")
    return tok


def check_page_table(page_indices, page_indptr, kv_last_page_len, page_size: int, pool_rows: int,
                     row_bytes: int = PACKED_BYTES):
    """Host-side guard for page tables: int32 contiguous device page numbers
    covering page_indptr[-1] entries, every row read inside the pool (a last
    page needs only its valid rows), and a pool small enough for 32-bit
    offsets (reads the pages back, one synchronisation)."""
    import torch
    if page_indices.dtype != torch.int32 or page_indices.dim() != 1 or not page_indices.is_contiguous():
        raise ValueError("page_indices must be a contiguous int32 tensor")
    pi = [int(v) for v in page_indptr]
    last = [int(v) for v in kv_last_page_len]
    if page_indices.numel() < pi[-1]:
        raise ValueError("page_indices is shorter than page_indptr[-1]")
    if pool_rows * row_bytes >= 2 ** 32:
        raise ValueError("the row pool must be smaller than 2^32 bytes")
    if pi[-1] > pi[0]:
        pages = page_indices[pi[0]:pi[-1]].to(torch.int64)
        # rows each page must hold: page_size, or the sequence's last-page count
        need = torch.full_like(pages, page_size)
        for b in range(len(last)):
            if pi[b + 1] > pi[b]:
                need[pi[b + 1] - 1 - pi[0]] = last[b]
        if int(pages.min()) < 0 or int((pages * page_size + need).max()) > pool_rows:
            raise ValueError("page_indices holds pages outside the pool")


def decode_mxfp4_24(q, kv_packed, kv_scale24, kv_indptr_dev, out, sm_scale: float, workspace, stream=None):
    """Enqueue the decode of the 24-scale MXFP4 cache (kv_scale24: uint8
    [T, 24], 8-byte aligned)."""
    _check(lib().mla_decode_mxfp4_24(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_packed.data_ptr()),
        ctypes.c_void_p(kv_scale24.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale), ctypes.c_void_p(workspace.data_ptr()),
        _stream_ptr(stream)), "mla_decode_mxfp4_24")


def decode_fp8(q, kv_fp8, kv_scale, kv_indptr_dev, out, sm_scale: float, workspace, stream=None):
    """Enqueue the fp8-cache decode (``kv_scale``: float32 [1] device tensor)."""
    _check(lib().mla_decode_fp8(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_fp8.data_ptr()),
        ctypes.c_void_p(kv_scale.data_ptr()), ctypes.c_void_p(kv_indptr_dev.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_float(sm_scale),
        ctypes.c_void_p(workspace.data_ptr()), _stream_ptr(stream)), "mla_decode_fp8")


def decode_bf16(q, kv_bf16, kv_indptr_dev, out, sm_scale: float, workspace, stream=None):
    """Enqueue the bf16-cache decode."""
    _check(lib().mla_decode_bf16(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_bf16.data_ptr()),
        ctypes.c_void_p(kv_indptr_dev.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_float(sm_scale), ctypes.c_void_p(workspace.data_ptr()), _stream_ptr(stream)),
        "mla_decode_bf16")


class MlaDecode:
    """Holds a planned workspace for one kv_indptr and runs decode calls.

    Tensors: q bf16 [B,16,576], kv_packed uint8 [T,288], kv_scale uint8
    [T,18], all on the same HIP device; ``kv_indptr`` is a host list/tensor.
    """

    def __init__(self, kv_indptr, device="cuda", num_cus: int = 0):
        import torch
        ind = [int(v) for v in kv_indptr]
        self.batch = len(ind) - 1
        self.indptr_host = ind
        self.device = torch.device(device)
        self.kv_indptr = torch.tensor(ind, dtype=torch.int32, device=self.device)
        total = ind[-1] - ind[0] if ind else 0
        nbytes = workspace_bytes(self.batch, total, num_cus)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        plan(ind, self.workspace, num_cus=num_cus)
        _release_on_free(self.workspace)

    def __call__(self, q, kv_packed, kv_scale, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        import torch
        if out is None:
            out = torch.empty(self.batch, NUM_HEADS, V_DIM, dtype=torch.bfloat16, device=self.device)
        _validate(q, kv_packed, kv_scale, out, self.batch)
        if kv_packed.shape[0] < self.indptr_host[-1]:
            raise ValueError("kv_indptr reaches past the end of the cache rows")
        decode(q, kv_packed, kv_scale, self.kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def mxfp4_24(self, q, kv_packed, kv_scale24, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        """Decode over the 24-scale MXFP4 cache: kv_packed uint8 [T,288],
        kv_scale24 uint8 [T,24] (byte k scales elements 24k..24k+23)."""
        import torch
        out = self._out(q, out)
        if kv_packed.dtype != torch.uint8 or kv_packed.dim() != 2 or kv_packed.shape[1] != PACKED_BYTES \
                or not kv_packed.is_contiguous():
            raise ValueError("kv_packed must be contiguous uint8 [T,288]")
        if kv_scale24.dtype != torch.uint8 or tuple(kv_scale24.shape) != (kv_packed.shape[0], 24) \
                or not kv_scale24.is_contiguous():
            raise ValueError("kv_scale24 must be contiguous uint8 [T,24]")
        if kv_packed.shape[0] < self.indptr_host[-1]:
            raise ValueError("kv_indptr reaches past the end of the cache rows")
        decode_mxfp4_24(q, kv_packed, kv_scale24, self.kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def mxfp4_paged(self, q, kv_packed, kv_scale, kv_indices, out=None, sm_scale=1.0 / math.sqrt(576.0),
                    stream=None, check=True):
        """Decode over row pools read through per-token indices (device int32
        tensor); ``check`` verifies the indices against the pool first."""
        import torch
        if out is None:
            out = torch.empty(self.batch, NUM_HEADS, V_DIM, dtype=torch.bfloat16, device=self.device)
        _validate(q, kv_packed, kv_scale, out, self.batch)
        if check:
            check_kv_indices(kv_indices, self.indptr_host, kv_packed.shape[0])
        decode_mxfp4_paged(q, kv_packed, kv_scale, kv_indices, self.kv_indptr, out, sm_scale, self.workspace,
                           stream)
        return out

    def fp8_paged(self, q, kv_fp8, kv_scale, kv_indices, out=None, sm_scale=1.0 / math.sqrt(576.0),
                  stream=None, check=True):
        """fp8 decode over a row pool read through per-token indices."""
        out = self._out(q, out)
        if check:
            check_kv_indices(kv_indices, self.indptr_host, kv_fp8.shape[0], QK_DIM)
        decode_fp8_paged(q, kv_fp8, kv_scale, kv_indices, self.kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def bf16_paged(self, q, kv_bf16, kv_indices, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None,
                   check=True):
        """bf16 decode over a row pool read through per-token indices."""
        out = self._out(q, out)
        if check:
            check_kv_indices(kv_indices, self.indptr_host, kv_bf16.shape[0], 2 * QK_DIM)
        decode_bf16_paged(q, kv_bf16, kv_indices, self.kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def _out(self, q, out):
        import torch
        if out is None:
            out = torch.empty(self.batch, NUM_HEADS, V_DIM, dtype=torch.bfloat16, device=self.device)
        _validate_qo(q, out, self.batch)
        return out

    def fp8(self, q, kv_fp8, kv_scale, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        """Decode over an fp8 cache: kv_fp8 uint8 E4M3 codes [T,576], kv_scale
        float32 [1] (per-tensor scale), both on the device."""
        out = self._out(q, out)
        _validate_dense("fp8", kv_fp8, kv_scale)
        if kv_fp8.shape[0] < self.indptr_host[-1]:
            raise ValueError("kv_indptr reaches past the end of the cache rows")
        decode_fp8(q, kv_fp8, kv_scale, self.kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def bf16(self, q, kv_bf16, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        """Decode over a bf16 cache: kv_bf16 bfloat16 [T,576] on the device."""
        out = self._out(q, out)
        _validate_dense("bf16", kv_bf16, None)
        if kv_bf16.shape[0] < self.indptr_host[-1]:
            raise ValueError("kv_indptr reaches past the end of the cache rows")
        decode_bf16(q, kv_bf16, self.kv_indptr, out, sm_scale, self.workspace, stream)
        return out


class MlaDecodePageTable:
    """A planned decode over a page table: sequence b owns pages
    ``page_indices[page_indptr[b]:page_indptr[b+1]]`` of ``page_size`` rows
    each, the last holding ``kv_last_page_len[b]`` valid rows; token t is
    pool row ``page * page_size + t % page_size`` of page ``t // page_size``.
    ``page_indptr`` and ``kv_last_page_len`` are host lists/tensors (the plan
    needs the token counts); the pools and ``page_indices`` are device
    tensors passed per call."""

    def __init__(self, page_indptr, kv_last_page_len, page_size: int, device="cuda", num_cus: int = 0):
        import torch
        tok = page_table_kv_indptr(page_indptr, kv_last_page_len, page_size)
        self.page_size = int(page_size)
        self.page_indptr_host = [int(v) for v in page_indptr]
        self.last_host = [int(v) for v in kv_last_page_len]
        self.plan = MlaDecode(tok, device=device, num_cus=num_cus)
        self.batch = self.plan.batch
        self.device = self.plan.device
        self.kv_indptr = self.plan.kv_indptr
        self.page_indptr = torch.tensor(self.page_indptr_host, dtype=torch.int32, device=self.device)

    def _run(self, fmt, q, pool, kv_scale, page_indices, out, sm_scale, stream, check, row_bytes):
        out = self.plan._out(q, out)
        if fmt == "mxfp4":
            _validate(q, pool, kv_scale, out, self.batch)
        else:
            _validate_dense(fmt, pool, kv_scale)
        if check:
            check_page_table(page_indices, self.page_indptr_host, self.last_host, self.page_size,
                             pool.shape[0], row_bytes)
        decode_page_table(fmt, q, pool, kv_scale, page_indices, self.page_indptr, self.page_size,
                          self.kv_indptr, out, sm_scale, self.plan.workspace, stream)
        return out

    def mxfp4(self, q, kv_packed, kv_scale, page_indices, out=None, sm_scale=1.0 / math.sqrt(576.0),
              stream=None, check=True):
        """MXFP4 decode: kv_packed uint8 [R,288], kv_scale uint8 [R,18] row pools."""
        return self._run("mxfp4", q, kv_packed, kv_scale, page_indices, out, sm_scale, stream, check,
                         PACKED_BYTES)

    def fp8(self, q, kv_fp8, kv_scale, page_indices, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None,
            check=True):
        """fp8 decode: kv_fp8 uint8 E4M3 [R,576], kv_scale float32 [1]."""
        return self._run("fp8", q, kv_fp8, kv_scale, page_indices, out, sm_scale, stream, check, QK_DIM)

    def bf16(self, q, kv_bf16, page_indices, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None,
             check=True):
        """bf16 decode: kv_bf16 bfloat16 [R,576]."""
        return self._run("bf16", q, kv_bf16, None, page_indices, out, sm_scale, stream, check, 2 * QK_DIM)


def group_entries(kv_indptr, groups: int):
    """Plan offsets and start rows of ``groups`` query entries per sequence:
    entry e = b * groups + g has sequence b's length and starts at its first
    row. Returns (entry offsets [B * groups + 1], start rows [B * groups])."""
    ind = [int(v) for v in kv_indptr]
    if groups < 1:
        raise ValueError("groups must be >= 1")
    entry, starts = [0], []
    for a, b in zip(ind, ind[1:]):
        for _ in range(groups):
            entry.append(entry[-1] + (b - a))
            starts.append(a)
    if entry[-1] >= 2 ** 31:
        raise ValueError("more than 2^31 - 1 tokens over all entries")
    return entry, starts


class MlaDecodeGroups:
    """A planned decode where every sequence of a contiguous cache serves
    ``groups`` consecutive 16-head query entries: entry e = b * groups + g
    reads the rows of sequence b (``kv_indptr`` on the host, as for
    ``MlaDecode``). q is bf16 [B * groups, 16, 576] and out bf16
    [B * groups, 16, 512]:
    * q_seq_len query tokens per sequence (token j of sequence b is entry
      b * q_seq_len + j): groups = q_seq_len;
    * 128 heads: q [B, 128, 576] viewed as [B * 8, 16, 576], groups = 8
      (both: groups = 8 * q_seq_len).
    Each entry is a full 16-head decode that reads the sequence's rows."""

    def __init__(self, kv_indptr, groups: int, device="cuda", num_cus: int = 0):
        import torch
        ind = [int(v) for v in kv_indptr]
        self.groups = int(groups)
        self.indptr_host = ind
        entry, starts = group_entries(ind, self.groups)
        if num_cus == 0:
            # up to one slot per entry (at most 4 per CU): the entries of a
            # sequence then hold consecutive slots that run at the same time
            # on one XCD and share its L2, instead of following each other
            # on one CU
            cus = _device_num_cus()
            num_cus = cus * max(1, min(4, -(-(len(entry) - 1) // cus)))
        self.num_cus = num_cus   # the slot count the plan spreads the entries over
        self.plan = MlaDecode(entry, device=device, num_cus=num_cus)
        self.batch = self.plan.batch
        self.device = self.plan.device
        self.kv_indptr = self.plan.kv_indptr
        self.kv_start = torch.tensor(starts if starts else [0], dtype=torch.int32, device=self.device)

    def _run(self, fmt, q, pool, kv_scale, out, sm_scale, stream):
        # [B, 16 * g, 576] (e.g. 128 heads) and [B * g, 16, 576] are the same memory
        if q.is_contiguous() and q.numel() == self.batch * NUM_HEADS * QK_DIM:
            q = q.view(self.batch, NUM_HEADS, QK_DIM)
        if out is not None and out.is_contiguous() and out.numel() == self.batch * NUM_HEADS * V_DIM:
            out = out.view(self.batch, NUM_HEADS, V_DIM)
        out = self.plan._out(q, out)
        if fmt == "mxfp4":
            _validate(q, pool, kv_scale, out, self.batch)
        else:
            _validate_dense(fmt, pool, kv_scale)
        if pool.shape[0] < self.indptr_host[-1]:
            raise ValueError("kv_indptr reaches past the end of the cache rows")
        decode_starts(fmt, q, pool, kv_scale, self.kv_start, self.kv_indptr, out, sm_scale, self.plan.workspace,
                      stream)
        return out

    def mxfp4(self, q, kv_packed, kv_scale, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        return self._run("mxfp4", q, kv_packed, kv_scale, out, sm_scale, stream)

    def fp8(self, q, kv_fp8, kv_scale, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        return self._run("fp8", q, kv_fp8, kv_scale, out, sm_scale, stream)

    def bf16(self, q, kv_bf16, out=None, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        return self._run("bf16", q, kv_bf16, None, out, sm_scale, stream)


class MlaDecodeDevicePlan:
    """Decode whose plan is built on the GPU from a device ``kv_indptr``
    tensor, for any offsets of ``batch`` sequences with at most
    ``max_total_kv`` tokens. ``plan(kv_indptr)`` and ``decode(...)`` only
    enqueue kernels, so a sequence of them can be captured in a HIP graph.
    """

    def __init__(self, batch: int, max_total_kv: int, device="cuda", num_cus: int = 0):
        import torch
        self.batch = batch
        self.max_total_kv = max_total_kv
        self.num_cus = num_cus
        self.device = torch.device(device)
        nbytes = workspace_bytes(batch, max_total_kv, num_cus)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        _release_on_free(self.workspace)

    def plan(self, kv_indptr, stream=None):
        import torch
        if kv_indptr.dtype != torch.int32 or tuple(kv_indptr.shape) != (self.batch + 1,) \
                or not kv_indptr.is_contiguous() or kv_indptr.device.type != "cuda":
            raise ValueError(f"kv_indptr must be a contiguous int32 device tensor [{self.batch + 1}]")
        plan_device(kv_indptr, self.batch, self.max_total_kv, self.workspace, self.num_cus, stream)

    def decode(self, q, kv_packed, kv_scale, kv_indptr, out, sm_scale=1.0 / math.sqrt(576.0),
               stream=None):
        _validate(q, kv_packed, kv_scale, out, self.batch)
        decode(q, kv_packed, kv_scale, kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def decode_paged(self, fmt, q, pool, kv_scale, kv_indices, kv_indptr, out,
                     sm_scale=1.0 / math.sqrt(576.0), stream=None):
        """Row-list decode on the device plan: fmt "mxfp4" (pool = packed rows,
        kv_scale = E8M0 rows), "fp8" (kv_scale = float32 [1]) or "bf16"
        (kv_scale unused). The indices are not checked (they may change on
        the device between graph replays): the caller keeps them in range."""
        _validate_qo(q, out, self.batch)
        if fmt == "mxfp4":
            decode_mxfp4_paged(q, pool, kv_scale, kv_indices, kv_indptr, out, sm_scale, self.workspace, stream)
        elif fmt == "fp8":
            decode_fp8_paged(q, pool, kv_scale, kv_indices, kv_indptr, out, sm_scale, self.workspace, stream)
        elif fmt == "bf16":
            decode_bf16_paged(q, pool, kv_indices, kv_indptr, out, sm_scale, self.workspace, stream)
        else:
            raise ValueError(f"unknown cache format {fmt!r}")
        return out

    def decode_page_table(self, fmt, q, pool, kv_scale, page_indices, page_indptr, page_size: int, kv_indptr,
                          out, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        """Page-table decode on the device plan (``kv_indptr``: the device
        token offsets the plan was built from; ``page_indptr``: the device
        page offsets). Nothing is checked (the tables may change on the
        device between graph replays): the caller keeps them consistent."""
        _validate_qo(q, out, self.batch)
        if fmt not in ("mxfp4", "fp8", "bf16"):
            raise ValueError(f"unknown cache format {fmt!r}")
        decode_page_table(fmt, q, pool, kv_scale, page_indices, page_indptr, page_size, kv_indptr, out, sm_scale,
                          self.workspace, stream)
        return out

    def decode_starts(self, fmt, q, pool, kv_scale, kv_start, kv_indptr, out, sm_scale=1.0 / math.sqrt(576.0),
                      stream=None):
        """Shared-row decode on the device plan: entry b reads its
        ``kv_indptr`` length of rows from row ``kv_start[b]`` on (device
        int32). Nothing is checked (the arrays may change on the device
        between graph replays): the caller keeps the rows in the cache."""
        _validate_qo(q, out, self.batch)
        if fmt not in ("mxfp4", "fp8", "bf16"):
            raise ValueError(f"unknown cache format {fmt!r}")
        decode_starts(fmt, q, pool, kv_scale, kv_start, kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def decode_fp8(self, q, kv_fp8, kv_scale, kv_indptr, out, sm_scale=1.0 / math.sqrt(576.0),
                   stream=None):
        """fp8-cache decode on the device plan (kv_fp8 uint8 [T,576], kv_scale float32 [1])."""
        _validate_qo(q, out, self.batch)
        decode_fp8(q, kv_fp8, kv_scale, kv_indptr, out, sm_scale, self.workspace, stream)
        return out

    def decode_bf16(self, q, kv_bf16, kv_indptr, out, sm_scale=1.0 / math.sqrt(576.0), stream=None):
        """bf16-cache decode on the device plan (kv_bf16 bfloat16 [T,576])."""
        _validate_qo(q, out, self.batch)
        decode_bf16(q, kv_bf16, kv_indptr, out, sm_scale, self.workspace, stream)
        return out


def _validate_qo(q, out, batch):
    import torch
    if q.dtype != torch.bfloat16 or tuple(q.shape) != (batch, NUM_HEADS, QK_DIM) or not q.is_contiguous():
        raise ValueError(f"q must be contiguous bf16 [{batch},16,576], got {q.dtype} {tuple(q.shape)}")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (batch, NUM_HEADS, V_DIM) or not out.is_contiguous():
        raise ValueError("out must be contiguous bf16 [B,16,512]")


def _validate_dense(fmt, pool, kv_scale):
    """fp8: uint8 (or float8_e4m3fn) rows [R,576] and a one-element float32
    scale on the same device; bf16: bfloat16 rows [R,576]."""
    import torch
    if fmt == "fp8":
        if pool.dtype not in (torch.uint8, torch.float8_e4m3fn) or pool.dim() != 2 \
                or pool.shape[1] != QK_DIM or not pool.is_contiguous():
            raise ValueError("kv_fp8 must be contiguous uint8/float8_e4m3fn [rows,576]")
        if kv_scale.dtype != torch.float32 or kv_scale.numel() != 1 or kv_scale.device != pool.device:
            raise ValueError("kv_scale must be a float32 device tensor of one element")
    elif pool.dtype != torch.bfloat16 or pool.dim() != 2 or pool.shape[1] != QK_DIM or not pool.is_contiguous():
        raise ValueError("kv_bf16 must be contiguous bfloat16 [rows,576]")


def _validate(q, kv_packed, kv_scale, out, batch):
    import torch
    if q.dtype != torch.bfloat16 or tuple(q.shape) != (batch, NUM_HEADS, QK_DIM) or not q.is_contiguous():
        raise ValueError(f"q must be contiguous bf16 [{batch},16,576], got {q.dtype} {tuple(q.shape)}")
    if kv_packed.dtype != torch.uint8 or kv_packed.dim() != 2 or kv_packed.shape[1] != PACKED_BYTES \
            or not kv_packed.is_contiguous():
        raise ValueError("kv_packed must be contiguous uint8 [T,288]")
    if kv_scale.dtype != torch.uint8 or tuple(kv_scale.shape) != (kv_packed.shape[0], SCALES_PER_TOKEN) \
            or not kv_scale.is_contiguous():
        raise ValueError("kv_scale must be contiguous uint8 [T,18]")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (batch, NUM_HEADS, V_DIM) or not out.is_contiguous():
        raise ValueError("out must be contiguous bf16 [B,16,512]")
