"""Reference append of new tokens' K/V into a paged cache (test infrastructure only).

Chunked prefill appends the new tokens of a request after its cached ones
before attention runs over the whole sequence [FI-0.6, kernel types:
Prefill].  Reading taken: the ``n_r`` new tokens of request ``r`` become
the last ``n_r`` tokens of its sequence once appended, so new token ``i``
lands at logical position ``kv_len_after[r] - n_r + i``, which the
block-sparse layout maps to page ``page_indices[page_indptr[r] + pos //
page_size]``, slot ``pos % page_size`` [FI-paper, methodology 1].  The
operation is a pure copy, so the reference is exact (byte for byte).
"""
from __future__ import annotations

import numpy as np


def append_paged_kv(k_pool, v_pool, page_indptr, page_indices, page_size, append_indptr, kv_len_after,
                    k_new, v_new, layout="HND"):
    """Return copies of the pools with the new tokens written in.

    k_pool/v_pool: [num_pages, Hk, page_size, d] ("HND") or [num_pages, page_size, Hk, d] ("NHD").
    append_indptr: [batch + 1] offsets of each request's new tokens in k_new/v_new [n_total, Hk, d].
    kv_len_after: [batch] sequence lengths including the new tokens.

    Pinned by: gathering the appended cache gives the old prefix followed by the new tokens; every
    slot that is not written keeps its old bytes; two appends in a row equal one append of both
    (tests)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    append_indptr = np.asarray(append_indptr, dtype=np.int64)
    for r in range(len(append_indptr) - 1):
        a, b = int(append_indptr[r]), int(append_indptr[r + 1])
        n = b - a
        for i in range(n):
            pos = int(kv_len_after[r]) - n + i
            page = int(page_indices[int(page_indptr[r]) + pos // page_size])
            slot = pos % page_size
            if layout == "HND":
                k_out[page, :, slot, :] = k_new[a + i]
                v_out[page, :, slot, :] = v_new[a + i]
            elif layout == "NHD":
                k_out[page, slot, :, :] = k_new[a + i]
                v_out[page, slot, :, :] = v_new[a + i]
            else:
                raise ValueError(layout)
    return k_out, v_out
