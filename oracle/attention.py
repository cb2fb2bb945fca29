"""fp64 reference attention over a paged / block-sparse KV cache (test infrastructure only).

What is computed, and the reading taken where the pages leave it open:

* KV as a block-sparse matrix [FI-paper, methodology 1; FI-0.6, architecture 1]:
  a request's logical KV sequence is its list of pages, in order; token j of
  request r lives in page ``page_indices[page_indptr[r] + j // page_size]``,
  slot ``j % page_size``.  A dense segment is the same with one contiguous
  block (``dense[kv_indptr[r] + j]``).
* Attention is plain scaled dot-product softmax attention, evaluated in
  fp64 from the stored (fp32 or bf16) values: s_ij = sm_scale * <q_i, k_j>,
  LSE_i = ln sum_{j visible} exp(s_ij), O_i = sum_j exp(s_ij - LSE_i) v_j.
  The pages name an ``lse`` output [FI-PR5329, code analysis 2] without
  its base; the natural log is taken.
* GQA [FI-0.6, kernel types: Decode]: q head ``hq`` reads kv head
  ``hq // (Hq / Hk)`` (consecutive groups).
* Query positions: the ``qo_len`` queries of a request are the last
  ``qo_len`` tokens of its own KV sequence (chunked prefill appends after
  cached KV [FI-0.6, kernel types: Prefill]), so query i sits at
  ``qpos = kv_len - qo_len + i``; the causal mask is aligned to it.
* Sliding window + attention sinks [FI-0.6, kernel types: Blackwell
  CuTe-DSL GQA decode]: key j is visible to a query at qpos iff it is in
  the window (``qpos - j < window``) or is one of the first ``sink``
  tokens; the union is taken, nothing counted twice.
* Fused RoPE [FI-paper, results: long-context Streaming-LLM and the fused
  RoPE + attention kernel]: rotate-half pairs (k, k + d/2) with angle
  ``pos * theta^(-2k/d)``; q and k are both rotated.  With K cached
  unrotated, "streaming" positions are ranks within the query's visible
  set (sinks then window, ascending); "absolute" uses j and qpos.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass
class PagedKV:
    """Paged cache: pools [num_pages, Hk, page_size, d] ("HND") or
    [num_pages, page_size, Hk, d] ("NHD")."""
    k_pool: np.ndarray
    v_pool: np.ndarray
    page_indptr: np.ndarray
    page_indices: np.ndarray
    page_size: int
    layout: str = "HND"


@dataclasses.dataclass
class DenseKV:
    """Contiguous cache [N, Hk, d]; request r owns rows [indptr[r], indptr[r+1])."""
    k: np.ndarray
    v: np.ndarray
    indptr: np.ndarray


def gather_kv(kv, r: int, tokens: np.ndarray):
    """K and V rows of request ``r`` for the given logical token indices, as fp64 [n, Hk, d].

    Block-sparse gather: page id from the request's page list, then the
    slot inside the page.  Pinned by: page-pool permutation invariance and
    paged == dense equality on the same logical sequence (tests)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    if isinstance(kv, DenseKV):
        rows = int(kv.indptr[r]) + tokens
        return kv.k[rows].astype(np.float64), kv.v[rows].astype(np.float64)
    pages = kv.page_indices[int(kv.page_indptr[r]) + tokens // kv.page_size].astype(np.int64)
    slots = tokens % kv.page_size
    if kv.layout == "HND":
        k = kv.k_pool[pages, :, slots, :]
        v = kv.v_pool[pages, :, slots, :]
    elif kv.layout == "NHD":
        k = kv.k_pool[pages, slots, :, :]
        v = kv.v_pool[pages, slots, :, :]
    else:
        raise ValueError(kv.layout)
    return k.astype(np.float64), v.astype(np.float64)


def visible(qpos: int, j: np.ndarray, kv_len: int, causal: bool, window: int, sink: int) -> np.ndarray:
    """Key visibility for one query: in range, causal (j <= qpos), and inside the
    sliding window or among the sink tokens."""
    j = np.asarray(j, dtype=np.int64)
    ok = (j >= 0) & (j < kv_len)
    if causal:
        ok &= j <= qpos
    if window > 0:
        ok &= ((qpos - j) < window) | (j < sink)
    return ok


def key_positions(qpos: int, vis_keys: np.ndarray, mode: str):
    """RoPE positions of the visible keys (ascending array) and of the query.

    "absolute": the token indices themselves.  "streaming": each visible
    key's rank inside the sorted visible set, and the query's rank; this
    keeps positions bounded by sink + window however long the cache is."""
    vis_keys = np.asarray(vis_keys, dtype=np.int64)
    if mode == "absolute":
        return vis_keys.copy(), int(qpos)
    if mode == "streaming":
        order = np.arange(len(vis_keys), dtype=np.int64)
        qrank = int(np.searchsorted(vis_keys, qpos))  # qpos is the last visible key under causal masking
        return order, qrank
    raise ValueError(mode)


def rope_rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x [..., d] at integer positions ``pos`` (broadcast over x[..., 0]).

    x'_k = x_k cos(a_k) - x_{k+d/2} sin(a_k);  x'_{k+d/2} = x_{k+d/2} cos(a_k) + x_k sin(a_k),
    a_k = pos * theta^(-2k/d), k < d/2.  Pinned by: the complex-multiplication form,
    norm preservation, identity at pos 0 and relative-position invariance (tests)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Store real values in bfloat16, round to nearest, ties to even, returned as fp64.

    bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of an IEEE
    binary32 number.  The value is rounded to binary32 first and then to bfloat16, the two
    roundings a value computed in binary32 and stored as bfloat16 goes through: the low 16
    bits of the binary32 pattern are rounded away by adding half of the dropped unit, minus
    one unless the kept part is odd (ties to even), and clearing them.  Finite inputs whose
    rounding stays finite only.  Pinned by: torch's own float32 -> bfloat16 conversion,
    ties included (tests)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    bits = x32.view(np.uint32).astype(np.uint64)
    keep_odd = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + keep_odd) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def _softmax_rows(s: np.ndarray, allowed: np.ndarray, v: np.ndarray):
    """Masked softmax attention for logits s [..., n], mask [..., n], values v [n, d].
    Rows with nothing visible get O = 0, LSE = -inf."""
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=-1, keepdims=True) if s.shape[-1] else np.full(s.shape[:-1] + (1,), -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.where(allowed, np.exp(s - m_safe), 0.0)
    l = p.sum(axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
        o = np.where(empty, 0.0, (p @ v) / np.where(empty, 1.0, l))
    return o, lse[..., 0]


def _attend_request(q_r, qpos, kv, r, kv_len, h, g, sm_scale, causal, window, sink, rope, theta,
                    kv_lo=0, kv_hi=None, block=256):
    """Rows of one request and one kv head: q_r [n, g', d] (the group's q heads), qpos [n].
    Keys restricted to [kv_lo, kv_hi) for partial states.  Returns O [n, g', d], LSE [n, g']."""
    n = q_r.shape[0]
    kv_hi = kv_len if kv_hi is None else kv_hi
    d = q_r.shape[-1]
    O = np.zeros((n,) + q_r.shape[1:], dtype=np.float64)
    L = np.full((n, q_r.shape[1]), -np.inf)
    all_j = np.arange(kv_len, dtype=np.int64)
    step = 1 if rope != "none" else block
    for a0 in range(0, n, step):
        a1 = min(n, a0 + step)
        vis = np.stack([visible(int(qpos[a]), all_j, kv_len, causal, window, sink) for a in range(a0, a1)])
        in_range = (all_j >= kv_lo) & (all_j < kv_hi)
        use = vis & in_range
        J = np.nonzero(use.any(axis=0))[0]
        if len(J) == 0:
            continue
        K, V = gather_kv(kv, r, J)
        K, V = K[:, h, :], V[:, h, :]
        qb = q_r[a0:a1]
        if rope != "none":
            vis_keys = np.nonzero(vis[0])[0]
            pk_all, pq = key_positions(int(qpos[a0]), vis_keys, rope)
            pk = pk_all[np.searchsorted(vis_keys, J)]
            K = rope_rotate(K, pk, theta)
            qb = rope_rotate(qb, np.full(qb.shape[:-1], pq), theta)
        # all rows of the block against all gathered keys as one matrix product (a library
        # primitive: the inner products of the definition, summed in BLAS order)
        s = sm_scale * (qb.reshape(-1, d) @ K.T).reshape(qb.shape[:-1] + (len(J),))
        o, lse = _softmax_rows(s, use[:, None, J], V)
        O[a0:a1] = o
        L[a0:a1] = lse
    return O, L


def attention(q, qo_indptr, kv_len, kv, num_kv_heads, sm_scale, causal=False, window=0, sink=0,
              rope="none", rope_theta=10000.0, tokens: Optional[Sequence[int]] = None):
    """Batched attention, every query token against its own request's KV.

    q [T, Hq, d] (float32 values, upcast exactly), outputs O [T, Hq, d] and
    LSE [T, Hq] in fp64.  ``tokens``: optional subset of global query token
    indices to evaluate (others are NaN) for sampled checks at full size.
    Pinned by: torch SDPA in fp64 (with its own causal mask on the
    equivalent full-prefill problem), closed forms, and an LSE probe key
    (tests)."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    g = Hq // num_kv_heads
    O = np.full((T, Hq, d), np.nan)
    L = np.full((T, Hq), np.nan)
    want = None if tokens is None else np.zeros(T, dtype=bool)
    if want is not None:
        want[np.asarray(tokens, dtype=np.int64)] = True
    for r in range(len(kv_len)):
        t0, t1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        n = t1 - t0
        if n == 0:
            continue
        Lr = int(kv_len[r])
        sel = np.arange(n) if want is None else np.nonzero(want[t0:t1])[0]
        if len(sel) == 0:
            continue
        qpos = Lr - n + sel
        for h in range(num_kv_heads):
            heads = slice(h * g, (h + 1) * g)
            o, lse = _attend_request(q[t0 + sel, heads, :], qpos, kv, r, Lr, h, g, sm_scale,
                                     causal, window, sink, rope, rope_theta)
            O[t0 + sel, heads, :] = o
            L[t0 + sel, heads] = lse
    return O, L


def attention_rope_stored(q, qo_indptr, kv_len, kv, num_kv_heads, sm_scale, window, sink, rope, rope_theta,
                          store=round_to_bf16):
    """RoPE attention as an unfused pipeline computes it: rotate, store, then plain attention.

    Reading taken for the unfused reference point of the fused RoPE kernel [FI-paper, results:
    fused RoPE + attention kernel]: a separate pass rotates every decode query (one per
    request, its last token at qpos = kv_len - 1) and the keys that query sees (causal, window
    plus sinks), at the positions ``key_positions`` gives, and writes them back in the cache's
    element type; the attention pass then reads those stored values with no rotation of its
    own.  Here the rotation is exact (``rope_rotate`` in fp64) and ``store`` is the storage
    rounding (bf16 round to nearest even by default); the softmax is as in ``attention``.
    Returns O [T, Hq, d] and LSE [T, Hq].  Pinned by: with ``store`` the identity it equals
    ``attention(..., rope=mode)`` (tests)."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    g = Hq // num_kv_heads
    O = np.full((T, Hq, d), np.nan)
    L = np.full((T, Hq), np.nan)
    for r in range(len(kv_len)):
        t0, t1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        if t1 == t0:
            continue
        assert t1 - t0 == 1, "the unfused reading rotates one decode query per request"
        Lr = int(kv_len[r])
        qpos = Lr - 1
        vis = np.nonzero(visible(qpos, np.arange(Lr), Lr, True, window, sink))[0]
        kpos, pq = key_positions(qpos, vis, rope)
        K, V = gather_kv(kv, r, vis)                                   # [n, Hk, d]
        Ks = store(rope_rotate(K, kpos[:, None], rope_theta))
        qs = store(rope_rotate(q[t0], np.full(Hq, pq), rope_theta))    # [Hq, d]
        for h in range(num_kv_heads):
            heads = slice(h * g, (h + 1) * g)
            s = sm_scale * (qs[heads] @ Ks[:, h, :].T)                 # [g, n]
            o, lse = _softmax_rows(s, np.ones(s.shape, dtype=bool), V[:, h, :])
            O[t0, heads] = o
            L[t0, heads] = lse
    return O, L


def attention_partial(q, qo_indptr, kv_len, kv, num_kv_heads, sm_scale, r, h, row_lo, row_hi,
                      kv_lo, kv_hi, causal=False, window=0, sink=0, rope="none", rope_theta=10000.0):
    """Partial state (O_c, LSE_c) of one work item: request r, kv head h, rows
    [row_lo, row_hi) of the request's (token, group-member) rows (row = i*g + u),
    keys restricted to [kv_lo, kv_hi).  Returns O [rows, d], LSE [rows]."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    g = Hq // num_kv_heads
    t0, t1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
    n = t1 - t0
    Lr = int(kv_len[r])
    rows = np.arange(row_lo, row_hi)
    i, u = rows // g, rows % g
    O = np.zeros((len(rows), d))
    L = np.full(len(rows), -np.inf)
    for a, (ii, uu) in enumerate(zip(i, u)):
        o, lse = _attend_request(q[t0 + ii, h * g + uu][None, None, :], np.array([Lr - n + ii]), kv, r, Lr, h,
                                 g, sm_scale, causal, window, sink, rope, rope_theta, kv_lo=kv_lo, kv_hi=kv_hi)
        O[a], L[a] = o[0, 0], lse[0, 0]
    return O, L


def merge(parts):
    """Combine partial states over a disjoint cover of the visible keys.

    M = max_c LSE_c;  LSE = M + ln sum_c exp(LSE_c - M);  O = sum_c exp(LSE_c - LSE) O_c.
    All partials empty (LSE = -inf) gives O = 0, LSE = -inf.  This is the
    split-KV state combination [FI-0.6, kernel types: split_kv]; pinned by
    split-then-merge == unsplit (tests).  parts: list of (O [..., d], LSE [...])."""
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    M = lses.max(axis=0)
    empty = ~np.isfinite(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp(lses - Ms)                         # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, tot)))
    scale = np.where(empty, 0.0, 1.0) * np.exp(lses - np.where(empty, 0.0, lse))
    o = (scale[..., None] * outs).sum(axis=0)
    return o, lse


def composable(q, prefix_kv: DenseKV, prefix_len: int, suffix_kv: PagedKV, suffix_len, num_kv_heads, sm_scale,
               tokens=None):
    """Shared-prefix parallel generation in the composable format [FI-paper,
    methodology 1]: the dense shared prefix and each branch's paged suffix
    are attended separately and their states merged.

    Branch b's single query token (q[b]) is the last token of its suffix;
    the whole prefix is in its past (no mask).  Pinned by equality with
    the flat layout (tests)."""
    B = len(suffix_len)
    op, lp = attention(q, np.array([0, B]), np.array([prefix_len]), prefix_kv, num_kv_heads, sm_scale,
                       causal=False, tokens=tokens)
    os_, ls = attention(q, np.arange(B + 1), np.asarray(suffix_len), suffix_kv, num_kv_heads, sm_scale,
                        causal=True, tokens=tokens)
    return merge([(op, lp), (os_, ls)])


def flat_from_composable(prefix_k, prefix_v, suffix_kv: PagedKV, suffix_len):
    """Flat paged layout of a composable batch: the prefix cut into pages that every
    branch's page list shares, followed by the branch's own suffix pages.
    prefix_k/v: [P, Hk, d] with P a multiple of the page size (HND pools).
    Returns (PagedKV, kv_len)."""
    ps = suffix_kv.page_size
    P, Hk, d = prefix_k.shape
    assert P % ps == 0 and suffix_kv.layout == "HND"
    npp = P // ps
    pk = prefix_k.reshape(npp, ps, Hk, d).transpose(0, 2, 1, 3)
    pv = prefix_v.reshape(npp, ps, Hk, d).transpose(0, 2, 1, 3)
    k_pool = np.concatenate([pk, suffix_kv.k_pool], axis=0)
    v_pool = np.concatenate([pv, suffix_kv.v_pool], axis=0)
    B = len(suffix_len)
    indptr = [0]
    idx = []
    for b in range(B):
        own = suffix_kv.page_indices[suffix_kv.page_indptr[b]:suffix_kv.page_indptr[b + 1]] + npp
        idx.extend(range(npp))
        idx.extend(own.tolist())
        indptr.append(len(idx))
    kv = PagedKV(k_pool, v_pool, np.asarray(indptr, dtype=np.int64), np.asarray(idx, dtype=np.int64), ps)
    return kv, np.asarray(suffix_len, dtype=np.int64) + P
