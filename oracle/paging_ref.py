"""Page tables for the CPU oracle (test infrastructure only; see the package
docstring).

Page "kernelbot-amd-mixed-mla-676098" (``_aiter_mla_decode``) calls its decode
with ``kv_indptr``, ``kv_indices``, ``kv_last_page_len`` and ``page_size``
(page size 1 there). Read with the usual page-table meaning: sequence b owns
the pages ``kv_indices[kv_indptr[b] : kv_indptr[b+1]]`` in that order, every
page is a run of ``page_size`` consecutive pool rows starting at
``page * page_size``, and only the first ``kv_last_page_len[b]`` rows of the
sequence's last page hold tokens. The sequence's tokens are those rows, page
by page, in order.
"""

import numpy as np


def page_table_rows(page_indices, page_indptr, kv_last_page_len, page_size: int):
    """Pool rows of every sequence of a page table, page by page: a list of
    int64 arrays (one per sequence, in token order)."""
    pages = np.asarray(page_indices, dtype=np.int64)
    pi = np.asarray(page_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    out = []
    for b in range(pi.shape[0] - 1):
        own = pages[int(pi[b]):int(pi[b + 1])]
        runs = []
        for j, page in enumerate(own):
            used = page_size if j + 1 < own.shape[0] else int(last[b])
            runs.append(page * page_size + np.arange(used, dtype=np.int64))
        out.append(np.concatenate(runs) if runs else np.zeros(0, dtype=np.int64))
    return out


def page_table_token_indptr(page_indptr, kv_last_page_len, page_size: int) -> np.ndarray:
    """Token offsets (from 0) of a page table's sequences."""
    pi = np.asarray(page_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    lens = [0 if pi[b + 1] == pi[b] else int((pi[b + 1] - pi[b] - 1) * page_size + last[b])
            for b in range(pi.shape[0] - 1)]
    return np.concatenate([[0], np.cumsum(lens, dtype=np.int64)])
