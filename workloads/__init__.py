"""Seeded synthetic inputs for paged / block-sparse batched attention.

This module holds no attention arithmetic: it only draws lengths, page
tables and N(0, 1) tensors, rounds them to the storage dtype and lays
them out.  Both the fp64 oracle (via the tests) and the HIP path are fed
from here, so the two see the same numbers.

Workloads follow the five shapes the problem statement names (a tiny
fp32 paged GQA decode, a Llama-3-8B-shaped decode, a ragged causal
prefill appended after cached KV, a shared-prefix parallel generation in
the composable dense+paged format, and a long-context streaming decode
with fused RoPE, sliding window and attention sinks).  The FlashInfer
pages measure on an unnamed "general serving benchmark"; these seeded
inputs stand in for it.

Random streams: every quantity has its own ``np.random.default_rng([seed,
stream])`` with stream 0 = lengths, 1 = page permutation, 2 = q, 3 = k,
4 = v, 5 = dense k, 6 = dense v.

KV pages are generated per *logical* page (request order, then page order
within the request) and scattered to physical pages by a random
permutation, so re-drawing the permutation leaves the logical KV sequence
of every request unchanged.  Token slots past ``kv_len`` in a request's
last page, pool pages no request references and (for windowed workloads)
pages no query can see are filled with NaN, so any read of them poisons
the result.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

LEN_STREAM, PERM_STREAM, Q_STREAM, K_STREAM, V_STREAM, DK_STREAM, DV_STREAM = range(7)


def rng_for(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32.

    NaN stays NaN.  Inputs here are finite N(0,1) draws or NaN poison, so
    the overflow-to-inf corner is never exercised."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.nan
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are already bf16-exact -> uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def lognormal_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """Integer lengths from a lognormal clipped to [lo, hi].

    The parameters put the clip bounds at +-2 sigma: mu is the log-midpoint
    and sigma a quarter of the log-range."""
    mu = 0.5 * (math.log(lo) + math.log(hi))
    sigma = (math.log(hi) - math.log(lo)) / 4.0
    z = rng.standard_normal(n)
    return np.clip(np.rint(np.exp(mu + sigma * z)), lo, hi).astype(np.int64)


def uniform_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi], both ends inclusive."""
    return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)


@dataclasses.dataclass
class Batch:
    """One batch of variable-length requests against a paged (or dense) KV cache.

    Shapes: q [T, Hq, d]; KV pages [*, Hk, page_size, d] ("HND": each
    (page, head) a contiguous page_size x d block).  All float arrays are
    float32 holding values exactly representable in ``dtype``."""

    name: str
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    qo_indptr: np.ndarray            # int32 [B+1]
    kv_len: np.ndarray               # int32 [B]
    causal: bool = False
    window: int = 0                  # <= 0: off
    sink: int = 0
    rope: str = "none"               # "none" | "streaming" | "absolute"
    rope_theta: float = 10000.0
    sm_scale: float = 0.0
    kv_mode: str = "paged"           # "paged" | "dense"
    # paged
    kv_page_indptr: Optional[np.ndarray] = None   # int32 [B+1] into kv_page_indices
    kv_page_indices: Optional[np.ndarray] = None  # int32 physical page ids
    num_pages: int = 0                            # physical pool size
    live_logical: Optional[np.ndarray] = None     # int64 logical page ids that hold data
    k_live: Optional[np.ndarray] = None           # [n_live, Hk, ps, d]
    v_live: Optional[np.ndarray] = None
    # dense
    kv_indptr: Optional[np.ndarray] = None        # int32 [B+1] token offsets into dense_k
    dense_k: Optional[np.ndarray] = None          # [N, Hk, d]
    dense_v: Optional[np.ndarray] = None
    q: Optional[np.ndarray] = None                # [T, Hq, d]

    @property
    def batch_size(self) -> int:
        return int(len(self.kv_len))

    @property
    def qo_len(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int64)

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    def host_pools(self):
        """Compact host view of the paged cache for the oracle.

        Returns (k_pool, v_pool, page_indices) where the pool holds the live
        logical pages in order plus one trailing all-NaN page, and
        page_indices maps every logical page to its slot (non-live pages to
        the NaN page).  This is a re-permutation of the physical pool, under
        which attention results do not change."""
        n_logical = int(self.kv_page_indptr[-1])
        n_live = len(self.live_logical)
        shape = (n_live + 1,) + self.k_live.shape[1:]
        kp = np.full(shape, np.nan, dtype=np.float32)
        vp = np.full(shape, np.nan, dtype=np.float32)
        kp[:n_live] = self.k_live
        vp[:n_live] = self.v_live
        remap = np.full(n_logical, n_live, dtype=np.int64)
        remap[self.live_logical] = np.arange(n_live)
        return kp, vp, remap.astype(np.int32)

    def physical_pools(self):
        """Full physical pool (host), NaN where no live page sits.  Small batches only."""
        shape = (self.num_pages,) + self.k_live.shape[1:]
        kp = np.full(shape, np.nan, dtype=np.float32)
        vp = np.full(shape, np.nan, dtype=np.float32)
        phys = self.kv_page_indices[self.live_logical]
        kp[phys] = self.k_live
        vp[phys] = self.v_live
        return kp, vp


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == BF16 else x.astype(np.float32)


def _normal(rng, shape, dtype):
    return _cast(rng.standard_normal(shape, dtype=np.float32), dtype)


def visible_token_ranges(kv_len, qo_len, causal, window, sink):
    """Per request, the union of key index ranges any of its queries may see,
    as a list of (lo, hi) half-open ranges.  Used only to decide which pages
    get data (the rest are NaN poison); the oracle applies the exact mask."""
    out = []
    for L, Q in zip(kv_len, qo_len):
        L, Q = int(L), int(Q)
        if window > 0:
            first_q = L - Q
            lo = max(0, first_q - window + 1)
            rngs = [(lo, L)]
            if lo > 0 and sink > 0:
                rngs.append((0, min(sink, lo)))
            out.append(rngs)
        else:
            out.append([(0, L)])
    return out


def paged_batch(*, name, seed, kv_len, qo_len, num_qo_heads, num_kv_heads, head_dim,
                page_size, dtype, pool_pages=None, causal=False, window=0, sink=0,
                rope="none", rope_theta=10000.0, sm_scale=None, perm_seed=None,
                poison_invisible=False) -> Batch:
    kv_len = np.asarray(kv_len, dtype=np.int64)
    qo_len = np.asarray(qo_len, dtype=np.int64)
    if qo_len.ndim == 0:
        qo_len = np.full(len(kv_len), int(qo_len), dtype=np.int64)
    B = len(kv_len)
    pages_per_req = (kv_len + page_size - 1) // page_size
    n_logical = int(pages_per_req.sum())
    num_pages = int(pool_pages) if pool_pages is not None else n_logical
    assert num_pages >= n_logical
    perm = rng_for(seed if perm_seed is None else perm_seed, PERM_STREAM).permutation(num_pages)
    kv_page_indices = perm[:n_logical].astype(np.int32)
    kv_page_indptr = np.zeros(B + 1, dtype=np.int32)
    kv_page_indptr[1:] = np.cumsum(pages_per_req)
    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_len)

    # live logical pages: every referenced page, or (poison_invisible) only those
    # holding a token some query may see
    live = []
    ranges = (visible_token_ranges(kv_len, qo_len, causal, window, sink) if poison_invisible
              else [[(0, int(L))] for L in kv_len])
    for r, rngs in enumerate(ranges):
        pages = set()
        for lo, hi in rngs:
            pages.update(range(lo // page_size, (hi - 1) // page_size + 1))
        live.extend(int(kv_page_indptr[r]) + p for p in sorted(pages))
    live_logical = np.asarray(sorted(live), dtype=np.int64)

    shape = (len(live_logical), num_kv_heads, page_size, head_dim)
    k_live = _normal(rng_for(seed, K_STREAM), shape, dtype)
    v_live = _normal(rng_for(seed, V_STREAM), shape, dtype)
    # poison token slots past kv_len in each request's last page
    req_of_page = np.searchsorted(kv_page_indptr, live_logical, side="right") - 1
    first_tok = (live_logical - kv_page_indptr[req_of_page]) * page_size
    for idx in range(len(live_logical)):
        valid = int(kv_len[req_of_page[idx]]) - int(first_tok[idx])
        if valid < page_size:
            k_live[idx, :, valid:, :] = np.nan
            v_live[idx, :, valid:, :] = np.nan

    T = int(qo_len.sum())
    q = _normal(rng_for(seed, Q_STREAM), (T, num_qo_heads, head_dim), dtype)
    return Batch(name=name, dtype=dtype, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, page_size=page_size, qo_indptr=qo_indptr,
                 kv_len=kv_len.astype(np.int32), causal=causal, window=window, sink=sink,
                 rope=rope, rope_theta=rope_theta,
                 sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim)),
                 kv_mode="paged", kv_page_indptr=kv_page_indptr, kv_page_indices=kv_page_indices,
                 num_pages=num_pages, live_logical=live_logical, k_live=k_live, v_live=v_live, q=q)


def dense_batch(*, name, seed, kv_len, qo_len, num_qo_heads, num_kv_heads, head_dim, dtype,
                causal=False, sm_scale=None, q=None) -> Batch:
    kv_len = np.asarray(kv_len, dtype=np.int64)
    qo_len = np.asarray(qo_len, dtype=np.int64)
    if qo_len.ndim == 0:
        qo_len = np.full(len(kv_len), int(qo_len), dtype=np.int64)
    B = len(kv_len)
    kv_indptr = np.zeros(B + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(kv_len)
    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_len)
    N = int(kv_len.sum())
    dk = _normal(rng_for(seed, DK_STREAM), (N, num_kv_heads, head_dim), dtype)
    dv = _normal(rng_for(seed, DV_STREAM), (N, num_kv_heads, head_dim), dtype)
    if q is None:
        q = _normal(rng_for(seed, Q_STREAM), (int(qo_len.sum()), num_qo_heads, head_dim), dtype)
    return Batch(name=name, dtype=dtype, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, page_size=1, qo_indptr=qo_indptr, kv_len=kv_len.astype(np.int32),
                 causal=causal, sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim)),
                 kv_mode="dense", kv_indptr=kv_indptr, dense_k=dk, dense_v=dv, q=q)


@dataclasses.dataclass
class Composable:
    """Shared-prefix parallel generation: one dense prefix + per-branch paged suffixes.

    ``prefix`` is a dense batch with one request whose queries are all the
    branch tokens (non-causal: the prefix lies in every branch's past);
    ``suffix`` is a paged decode batch, one request per branch, sharing the
    same q."""
    prefix: Batch
    suffix: Batch


# ---------------------------------------------------------------------------
# The five named workloads.  ``scale`` shrinks batch / lengths for fast tests.
# ---------------------------------------------------------------------------

def tiny_decode_f32(seed: int = 1, perm_seed=None) -> Batch:
    """4 requests, kv {17,64,130,255}, page_size 16, 64-page permuted pool, 8/2 heads, d 64, fp32."""
    return paged_batch(name="tiny_paged_gqa_decode_f32", seed=seed, kv_len=[17, 64, 130, 255], qo_len=1,
                       num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16, dtype=F32,
                       pool_pages=64, sm_scale=1.0 / 8.0, perm_seed=perm_seed)


def llama3_decode_lengths(seed: int = 2, batch: int = 64, lo: int = 512, hi: int = 8192):
    kv = lognormal_lengths(rng_for(seed, LEN_STREAM), batch, lo, hi)
    return np.ones(batch, dtype=np.int64), kv


def llama3_decode(seed: int = 2, batch: int = 64, lo: int = 512, hi: int = 8192, perm_seed=None) -> Batch:
    """Llama-3-8B-shaped decode layer: 32 q / 8 kv heads, d 128, bf16, page_size 16,
    kv lengths lognormal clipped to [lo, hi]."""
    _, kv = llama3_decode_lengths(seed, batch, lo, hi)
    return paged_batch(name="llama3_8b_paged_decode_bf16", seed=seed, kv_len=kv, qo_len=1,
                       num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=BF16,
                       perm_seed=perm_seed)


def ragged_prefill_lengths(seed: int = 3, batch: int = 16, q_lo: int = 128, q_hi: int = 4096,
                           p_lo: int = 0, p_hi: int = 2048):
    r = rng_for(seed, LEN_STREAM)
    qlen = lognormal_lengths(r, batch, q_lo, q_hi)
    plen = uniform_lengths(r, batch, p_lo, p_hi)
    return qlen, plen + qlen


def ragged_prefill(seed: int = 3, batch: int = 16, q_lo: int = 128, q_hi: int = 4096,
                   p_lo: int = 0, p_hi: int = 2048) -> Batch:
    """Ragged causal prefill appended after cached KV: new lengths lognormal [q_lo, q_hi],
    existing prefix uniform [p_lo, p_hi]; 32 q / 8 kv heads, d 128, bf16, page_size 16."""
    qlen, kvlen = ragged_prefill_lengths(seed, batch, q_lo, q_hi, p_lo, p_hi)
    plen = kvlen - qlen
    return paged_batch(name="ragged_causal_prefill_append_bf16", seed=seed, kv_len=plen + qlen, qo_len=qlen,
                       num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=BF16, causal=True)


def shared_prefix_lengths(seed: int = 4, branches: int = 64, s_lo: int = 128, s_hi: int = 1024):
    """Suffix lengths of the branches."""
    return uniform_lengths(rng_for(seed, LEN_STREAM), branches, s_lo, s_hi)


def shared_prefix(seed: int = 4, branches: int = 64, prefix_len: int = 16384,
                  s_lo: int = 128, s_hi: int = 1024) -> Composable:
    """Shared 16384-token dense prefix + 64 paged branch suffixes uniform [128, 1024],
    one decode token per branch; 32 q / 8 kv heads, d 128, bf16, page_size 16."""
    slen = shared_prefix_lengths(seed, branches, s_lo, s_hi)
    suffix = paged_batch(name="shared_prefix_suffix_bf16", seed=seed, kv_len=slen, qo_len=1,
                         num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=BF16,
                         causal=True)
    prefix = dense_batch(name="shared_prefix_dense_bf16", seed=seed, kv_len=[prefix_len], qo_len=[branches],
                         num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype=BF16, causal=False, q=suffix.q)
    return Composable(prefix=prefix, suffix=suffix)


def mixed_lengths(seed: int = 6, decode: int = 64, prefill: int = 4, d_lo: int = 512, d_hi: int = 8192,
                  q_lo: int = 256, q_hi: int = 2048, p_lo: int = 0, p_hi: int = 2048):
    """Continuous batching: `decode` one-token requests with lognormal [d_lo, d_hi] kv lengths and
    `prefill` chunk requests (lognormal [q_lo, q_hi] new tokens after a uniform [p_lo, p_hi] cached
    prefix), the prefill requests spread evenly through the batch."""
    r = rng_for(seed, LEN_STREAM)
    dkv = lognormal_lengths(r, decode, d_lo, d_hi)
    pq = lognormal_lengths(r, prefill, q_lo, q_hi)
    pp = uniform_lengths(r, prefill, p_lo, p_hi)
    qo = np.ones(decode + prefill, dtype=np.int64)
    kv = np.zeros(decode + prefill, dtype=np.int64)
    at = set(int(i) for i in np.linspace(0, decode + prefill - 1, prefill).round()) if prefill else set()
    di = pi = 0
    for i in range(decode + prefill):
        if i in at:
            qo[i], kv[i] = pq[pi], pp[pi] + pq[pi]
            pi += 1
        else:
            kv[i] = dkv[di]
            di += 1
    return qo, kv


def mixed(seed: int = 6, decode: int = 64, prefill: int = 4) -> Batch:
    """Mixed decode + prefill batch of one Llama-3-8B-shaped layer: 32 q / 8 kv heads, d 128, bf16,
    page_size 16, causal (see mixed_lengths)."""
    qo, kv = mixed_lengths(seed, decode, prefill)
    return paged_batch(name="mixed_decode_prefill_bf16", seed=seed, kv_len=kv, qo_len=qo, num_qo_heads=32,
                       num_kv_heads=8, head_dim=128, page_size=16, dtype=BF16, causal=True)


def streaming_rope_decode_lengths(seed: int = 5, batch: int = 8, lo: int = 32768, hi: int = 131072):
    kv = uniform_lengths(rng_for(seed, LEN_STREAM), batch, lo, hi)
    return np.ones(batch, dtype=np.int64), kv


def streaming_rope_decode(seed: int = 5, batch: int = 8, lo: int = 32768, hi: int = 131072,
                          window: int = 4096, sink: int = 4, rope: str = "streaming") -> Batch:
    """Long-context Streaming-LLM decode: kv uniform [lo, hi], 64 q / 8 kv heads, d 128, bf16,
    page_size 16, K cached unrotated, RoPE theta 5e5 applied in-kernel, window 4096 + 4 sinks."""
    _, kv = streaming_rope_decode_lengths(seed, batch, lo, hi)
    return paged_batch(name="streaming_rope_window_sink_decode_bf16", seed=seed, kv_len=kv, qo_len=1,
                       num_qo_heads=64, num_kv_heads=8, head_dim=128, page_size=16, dtype=BF16,
                       causal=True, window=window, sink=sink, rope=rope, rope_theta=500000.0,
                       poison_invisible=True)
