"""Test-side adapters: workloads.Batch -> oracle calls, and an independent
logical-KV route for library cross-checks.  Test infrastructure only."""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import DenseKV, PagedKV


def oracle_kv(b, physical: bool = False):
    if b.kv_mode == "dense":
        return DenseKV(b.dense_k, b.dense_v, b.kv_indptr)
    if physical:
        kp, vp = b.physical_pools()
        return PagedKV(kp, vp, b.kv_page_indptr, b.kv_page_indices, b.page_size)
    kp, vp, idx = b.host_pools()
    return PagedKV(kp, vp, b.kv_page_indptr, idx, b.page_size)


def oracle_attention(b, tokens=None, kv=None, **over):
    kw = dict(causal=b.causal, window=b.window, sink=b.sink, rope=b.rope, rope_theta=b.rope_theta)
    kw.update(over)
    return oracle.attention(b.q, b.qo_indptr, b.kv_len, kv if kv is not None else oracle_kv(b),
                            b.num_kv_heads, b.sm_scale, tokens=tokens, **kw)


def logical_kv(b, r):
    """Request r's K/V sequence [L, Hk, d] read straight from the generator's
    logical page order (no page table involved).  Needs every page of r live."""
    L = int(b.kv_len[r])
    if b.kv_mode == "dense":
        s = int(b.kv_indptr[r])
        return b.dense_k[s:s + L].astype(np.float64), b.dense_v[s:s + L].astype(np.float64)
    p0, p1 = int(b.kv_page_indptr[r]), int(b.kv_page_indptr[r + 1])
    pos = np.searchsorted(b.live_logical, np.arange(p0, p1))
    assert np.array_equal(b.live_logical[pos], np.arange(p0, p1)), "request has non-live pages"
    k = b.k_live[pos].transpose(0, 2, 1, 3).reshape(-1, b.num_kv_heads, b.head_dim)[:L]
    v = b.v_live[pos].transpose(0, 2, 1, 3).reshape(-1, b.num_kv_heads, b.head_dim)[:L]
    return k.astype(np.float64), v.astype(np.float64)


def sdpa(q, k, v, scale, is_causal=False, attn_mask=None):
    """torch scaled_dot_product_attention in fp64 on the CPU.
    q [n, Hq, d], k/v [L, Hk, d]; kv heads repeated per group (hq -> hq // g)."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=is_causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def oracle_attention_all(b, workers=None, token_chunk=512, kv=None):
    """oracle_attention on every query token of a large batch, evaluated by a thread pool.

    Each task is one request's tokens [a, a + token_chunk) (the request's full query block is
    passed, so query positions are those of the whole request); numpy's element-wise passes and
    BLAS release the GIL, and BLAS is held to one thread per task so the tasks do not
    oversubscribe the cores."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    kv = kv if kv is not None else oracle_kv(b)
    T, Hq, d = b.q.shape
    B = b.batch_size
    O = np.full((T, Hq, d), np.nan)
    L = np.full((T, Hq), np.nan)
    tasks = []
    for r in range(B):
        t0, t1 = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
        for a in range(t0, t1, token_chunk):
            cost = (min(t1, a + token_chunk) - a) * int(b.kv_len[r])
            tasks.append((cost, r, t0, t1, a, min(t1, a + token_chunk)))
    tasks.sort(reverse=True)

    def one(task):
        _, r, t0, t1, a, c = task
        n = t1 - t0
        qo = np.zeros(B + 1, dtype=np.int64)
        qo[r + 1:] = n  # request r owns rows [0, n) of the sub-array; every other request is empty
        o, l = oracle.attention(b.q[t0:t1], qo, b.kv_len, kv, b.num_kv_heads, b.sm_scale, causal=b.causal,
                                window=b.window, sink=b.sink, rope=b.rope, rope_theta=b.rope_theta,
                                tokens=range(a - t0, c - t0))
        return a, c, o[a - t0:c - t0], l[a - t0:c - t0]

    n_workers = workers or min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=1), ThreadPoolExecutor(n_workers) as ex:
        for a, c, o, l in ex.map(one, tasks):
            O[a:c] = o
            L[a:c] = l
    return O, L
