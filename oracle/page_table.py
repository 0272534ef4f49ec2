"""CSR page table (oracle).

Follows aicassindra "FlashInfer, in depth", section "The block-sparse page
table": request i owns entries indptr[i]..indptr[i+1] of ``indices`` (page ids
in token order), and ``last_page_len`` counts the filled slots of its final
page, from 1 to page_size.  The length identity l = P (n - 1) + r with
1 <= r <= P is the one on the pinghaoyang page, section "页表就是一张块稀疏矩阵"
(the page table is a block-sparse matrix).
"""

from __future__ import annotations

import numpy as np


def page_table(kv_lens, page_size: int, page_ids=None):
    """Build (indptr, indices, last_page_len) as int32 arrays.

    A request of l tokens needs the smallest n with n * P >= l pages; its last
    page then holds l - (n - 1) * P tokens.  Pages are handed out from
    ``page_ids`` (default 0, 1, 2, ...) in request order."""
    P = int(page_size)
    if P < 1:
        raise ValueError("page_size must be positive")
    lens = [int(x) for x in kv_lens]
    counts, lasts = [], []
    for length in lens:
        if length < 1:
            raise ValueError("a request must hold at least one token")
        n = length // P + (1 if length % P else 0)
        counts.append(n)
        lasts.append(length - (n - 1) * P)
    indptr = np.concatenate([[0], np.cumsum(counts, dtype=np.int64)]).astype(np.int32)
    nnz = int(indptr[-1])
    if page_ids is None:
        indices = np.arange(nnz, dtype=np.int32)
    else:
        page_ids = np.asarray(page_ids)
        if page_ids.shape[0] < nnz:
            raise ValueError("not enough page ids")
        indices = page_ids[:nnz].astype(np.int32)
    return indptr, indices, np.asarray(lasts, dtype=np.int32)


def kv_lengths(kv_indptr, kv_last_page_len, page_size: int) -> np.ndarray:
    """l_i = P (n_i - 1) + r_i with n_i = indptr[i+1] - indptr[i]."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    n = indptr[1:] - indptr[:-1]
    return page_size * (n - 1) + last


def check(kv_indptr, kv_last_page_len, page_size: int) -> None:
    """Raise ValueError unless the CSR is well formed: indptr starts at 0 and
    every request has at least one page whose fill r lies in [1, P]."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    if indptr.ndim != 1 or indptr.shape[0] != last.shape[0] + 1:
        raise ValueError("indptr must have batch + 1 entries")
    if indptr[0] != 0:
        raise ValueError("indptr[0] must be 0")
    if np.any(indptr[1:] - indptr[:-1] < 1):
        raise ValueError("every request needs at least one page")
    if np.any(last < 1) or np.any(last > page_size):
        raise ValueError("last_page_len must lie in [1, page_size]")
