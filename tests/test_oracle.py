"""Pins for the fp64 oracle: each check ties it to something other than itself
(torch's SDPA, closed forms, invariants, brute force, a committed golden plan)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.attention import DenseKV, PagedKV
from tests.helpers import logical_kv, oracle_attention, oracle_kv, sdpa

HERE = os.path.dirname(os.path.abspath(__file__))


def small_paged(seed=11, kv=(5, 16, 33, 70), qo=1, Hq=8, Hk=2, d=16, ps=4, dtype=W.F32, **kw):
    return W.paged_batch(name="t", seed=seed, kv_len=list(kv), qo_len=qo, num_qo_heads=Hq, num_kv_heads=Hk,
                         head_dim=d, page_size=ps, dtype=dtype, **kw)


# ---------------------------------------------------------------- core attention vs torch SDPA

@pytest.mark.parametrize("qo", [1, 3])
def test_noncausal_matches_sdpa(qo):
    b = small_paged(qo=qo)
    O, L = oracle_attention(b, causal=False)
    for r in range(b.batch_size):
        k, v = logical_kv(b, r)
        t0, t1 = b.qo_indptr[r], b.qo_indptr[r + 1]
        ref = sdpa(b.q[t0:t1], k, v, b.sm_scale)
        np.testing.assert_allclose(O[t0:t1], ref, rtol=0, atol=1e-12)


def test_full_prefill_causal_matches_sdpa():
    kv = (7, 16, 29)
    b = small_paged(kv=kv, qo=np.array(kv), causal=True, seed=12)
    O, _ = oracle_attention(b)
    for r in range(b.batch_size):
        k, v = logical_kv(b, r)
        t0, t1 = b.qo_indptr[r], b.qo_indptr[r + 1]
        ref = sdpa(b.q[t0:t1], k, v, b.sm_scale, is_causal=True)
        np.testing.assert_allclose(O[t0:t1], ref, rtol=0, atol=1e-12)


def test_append_equals_tail_of_full_prefill():
    """Causal prefill appended after cached KV: the new queries must equal the last
    rows of a full causal prefill over the whole sequence (SDPA's own mask)."""
    kv, qo = np.array([9, 40, 23]), np.array([3, 17, 1])
    b = small_paged(kv=kv, qo=qo, causal=True, seed=13)
    O, _ = oracle_attention(b)
    rng = np.random.default_rng(99)
    for r in range(b.batch_size):
        k, v = logical_kv(b, r)
        L, Q = int(kv[r]), int(qo[r])
        t0 = b.qo_indptr[r]
        full_q = rng.standard_normal((L, b.num_qo_heads, b.head_dim))
        full_q[L - Q:] = b.q[t0:t0 + Q]
        ref = sdpa(full_q, k, v, b.sm_scale, is_causal=True)[L - Q:]
        np.testing.assert_allclose(O[t0:t0 + Q], ref, rtol=0, atol=1e-12)


def test_lse_via_probe_key():
    """LSE pinned through SDPA: prepend a zero key (logit 0) whose value is a unit
    vector on an extra channel; that channel's output is 1 / (1 + exp(LSE))."""
    kv = (12, 31)
    b = small_paged(kv=kv, qo=np.array(kv), causal=True, seed=14)
    _, Lse = oracle_attention(b)
    for r in range(b.batch_size):
        k, v = logical_kv(b, r)
        L = int(kv[r])
        t0 = b.qo_indptr[r]
        Hk, d = b.num_kv_heads, b.head_dim
        k2 = np.concatenate([np.zeros((1, Hk, d)), k], axis=0)
        v2 = np.concatenate([np.zeros((L + 1, Hk, d)), np.zeros((L + 1, Hk, 1))], axis=2)
        v2[1:, :, :d] = v
        v2[0, :, d] = 1.0
        q2 = np.concatenate([np.zeros((1, b.num_qo_heads, d)), b.q[t0:t0 + L]], axis=0)
        o = sdpa(q2, k2, v2, b.sm_scale, is_causal=True)[1:, :, d]
        np.testing.assert_allclose(Lse[t0:t0 + L], np.log(1.0 / o - 1.0), rtol=0, atol=1e-9)


def test_gqa_mapping_against_per_head_sdpa():
    """q head hq reads kv head hq // g: compare one head at a time with a 1-head SDPA."""
    b = small_paged(kv=(21,), Hq=6, Hk=3, seed=15)
    O, _ = oracle_attention(b, causal=False)
    k, v = logical_kv(b, 0)
    for hq in range(6):
        ref = sdpa(b.q[:, hq:hq + 1], k[:, hq // 2:hq // 2 + 1], v[:, hq // 2:hq // 2 + 1], b.sm_scale)
        np.testing.assert_allclose(O[:, hq], ref[:, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_single_visible_key():
    b = small_paged(kv=(30, 9), causal=True, window=1, seed=16)
    O, L = oracle_attention(b)
    for r in range(b.batch_size):
        k, v = logical_kv(b, r)
        j = int(b.kv_len[r]) - 1
        for hq in range(b.num_qo_heads):
            np.testing.assert_array_equal(O[r, hq], v[j, hq // b.group])
            s = b.sm_scale * float(np.dot(b.q[r, hq].astype(np.float64), k[j, hq // b.group]))
            assert abs(L[r, hq] - s) < 1e-13


def test_zero_query_is_mean():
    b = small_paged(kv=(30, 9, 64), causal=True, seed=17)
    b.q[:] = 0
    O, L = oracle_attention(b)
    for r in range(b.batch_size):
        _, v = logical_kv(b, r)
        n = int(b.kv_len[r])
        np.testing.assert_allclose(O[r], v.mean(axis=0).repeat(b.group, axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[r], math.log(n), rtol=0, atol=1e-13)


def test_constant_values():
    b = small_paged(kv=(30, 9), causal=True, seed=18)
    b.v_live[:] = np.where(np.isnan(b.v_live), np.nan, 0.625)
    O, _ = oracle_attention(b)
    np.testing.assert_allclose(O, 0.625, rtol=0, atol=1e-14)


def test_window_and_sink_union():
    """window 1 + s sinks with q = 0: visible keys are {0..s-1} U {qpos}, equal weights."""
    s = 3
    b = small_paged(kv=(40, 2, 3), causal=True, window=1, sink=s, seed=19)
    b.q[:] = 0
    O, L = oracle_attention(b)
    for r in range(b.batch_size):
        _, v = logical_kv(b, r)
        n = int(b.kv_len[r])
        keys = sorted(set(range(min(s, n))) | {n - 1})
        np.testing.assert_allclose(O[r], v[keys].mean(axis=0).repeat(b.group, axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[r], math.log(len(keys)), rtol=0, atol=1e-13)


def test_wide_window_no_sink_is_causal():
    kv = np.array([20, 33])
    b = small_paged(kv=kv, qo=np.array([5, 33]), causal=True, window=64, sink=0, seed=20)
    O1, L1 = oracle_attention(b)
    O2, L2 = oracle_attention(b, window=0)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_window_prefill_against_sdpa_band_mask():
    """Windowed causal prefill against SDPA given an explicit band mask built from
    index differences (|window| keys ending at the query)."""
    kv = np.array([37])
    b = small_paged(kv=kv, qo=kv, causal=True, window=5, sink=0, seed=21)
    O, _ = oracle_attention(b)
    k, v = logical_kv(b, 0)
    i = np.arange(37)[:, None]
    j = np.arange(37)[None, :]
    band = (j <= i) & (j > i - 5)
    ref = sdpa(b.q, k, v, b.sm_scale, attn_mask=band)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- gather / layout invariants

def test_page_pool_permutation_invariance():
    b1 = small_paged(seed=22, pool_pages=64, perm_seed=100)
    b2 = small_paged(seed=22, pool_pages=64, perm_seed=200)
    assert not np.array_equal(b1.kv_page_indices, b2.kv_page_indices)
    O1, L1 = oracle_attention(b1, kv=oracle_kv(b1, physical=True))
    O2, L2 = oracle_attention(b2, kv=oracle_kv(b2, physical=True))
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)
    assert np.isfinite(O1).all()


def test_paged_equals_dense_and_nhd():
    b = small_paged(seed=23, kv=(13, 40))
    O1, L1 = oracle_attention(b, kv=oracle_kv(b, physical=True))
    ks, vs = zip(*[logical_kv(b, r) for r in range(b.batch_size)])
    dense = DenseKV(np.concatenate(ks), np.concatenate(vs), np.concatenate([[0], np.cumsum(b.kv_len)]))
    O2, L2 = oracle_attention(b, kv=dense)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)
    kp, vp = b.physical_pools()
    nhd = PagedKV(kp.transpose(0, 2, 1, 3).copy(), vp.transpose(0, 2, 1, 3).copy(), b.kv_page_indptr,
                  b.kv_page_indices, b.page_size, layout="NHD")
    O3, _ = oracle_attention(b, kv=nhd)
    np.testing.assert_array_equal(O1, O3)


# ---------------------------------------------------------------- split / merge

def test_random_split_merge_equals_unsplit():
    b = small_paged(seed=24, kv=(50, 77), qo=np.array([3, 5]), causal=True, window=20, sink=2)
    kv = oracle_kv(b)
    O, L = oracle_attention(b)
    rng = np.random.default_rng(5)
    g = b.group
    for r in range(b.batch_size):
        Lr = int(b.kv_len[r])
        cuts = np.sort(rng.choice(np.arange(1, Lr), size=4, replace=False))
        bounds = [0, *cuts.tolist(), Lr]
        rows = int(b.qo_len[r]) * g
        for h in range(b.num_kv_heads):
            parts = [oracle.attention_partial(b.q, b.qo_indptr, b.kv_len, kv, b.num_kv_heads, b.sm_scale, r, h, 0,
                                              rows, a, c, causal=True, window=20, sink=2)
                     for a, c in zip(bounds[:-1], bounds[1:])]
            o, l = oracle.merge(parts)
            t0 = b.qo_indptr[r]
            ref_o = O[t0:t0 + rows // g, h * g:(h + 1) * g].reshape(rows, -1)
            ref_l = L[t0:t0 + rows // g, h * g:(h + 1) * g].reshape(rows)
            np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


def test_merge_empty_and_single():
    o = np.arange(6.0).reshape(2, 3)
    l = np.array([0.5, -np.inf])
    mo, ml = oracle.merge([(o, l), (np.zeros((2, 3)), np.array([-np.inf, -np.inf]))])
    np.testing.assert_array_equal(mo[0], o[0])
    assert ml[0] == 0.5 and ml[1] == -np.inf
    np.testing.assert_array_equal(mo[1], 0.0)


def test_merge_two_halves_closed_form():
    """Two partials with equal LSE: output is their average, LSE + ln 2."""
    a, c = np.array([[1.0, 2.0]]), np.array([[3.0, -2.0]])
    mo, ml = oracle.merge([(a, np.array([1.25])), (c, np.array([1.25]))])
    np.testing.assert_allclose(mo, [[2.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(ml, [1.25 + math.log(2.0)], atol=1e-15)


# ---------------------------------------------------------------- composable format

def test_composable_equals_flat():
    c = W.shared_prefix(seed=25, branches=5, prefix_len=64, s_lo=3, s_hi=40)
    # small head count to keep it fast
    pre, suf = c.prefix, c.suffix
    kvp = DenseKV(pre.dense_k, pre.dense_v, pre.kv_indptr)
    kp, vp = suf.physical_pools()
    kvs = PagedKV(kp, vp, suf.kv_page_indptr, suf.kv_page_indices, suf.page_size)
    O1, L1 = oracle.composable(suf.q, kvp, 64, kvs, suf.kv_len, suf.num_kv_heads, suf.sm_scale)
    flat, flat_len = oracle.flat_from_composable(pre.dense_k, pre.dense_v, kvs, suf.kv_len)
    O2, L2 = oracle.attention(suf.q, suf.qo_indptr, flat_len, flat, suf.num_kv_heads, suf.sm_scale, causal=True)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- RoPE

def test_rope_complex_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 16))
    pos = np.arange(7) * 13
    y = oracle.rope_rotate(x, pos, 500000.0)
    z = (x[:, :8] + 1j * x[:, 8:]) * np.exp(1j * pos[:, None] * 500000.0 ** (-np.arange(0, 16, 2) / 16.0))
    np.testing.assert_allclose(y[:, :8], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 8:], z.imag, atol=1e-12)


def test_rope_identity_norm_relative():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64))
    np.testing.assert_array_equal(oracle.rope_rotate(q, 0, 1e4), q)
    y = oracle.rope_rotate(q, 12345, 5e5)
    assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
    a = np.dot(oracle.rope_rotate(q, 100, 5e5), oracle.rope_rotate(k, 37, 5e5))
    c = np.dot(oracle.rope_rotate(q, 100 + 999, 5e5), oracle.rope_rotate(k, 37 + 999, 5e5))
    assert abs(a - c) < 1e-10


def test_rope_absolute_against_sdpa():
    """Absolute-position RoPE attention = SDPA on explicitly rotated q and k."""
    kv = np.array([19, 33])
    b = small_paged(kv=kv, qo=1, causal=True, rope="absolute", rope_theta=500000.0, seed=26)
    O, _ = oracle_attention(b)
    for r in range(b.batch_size):
        k, v = logical_kv(b, r)
        L = int(kv[r])
        kr = oracle.rope_rotate(k, np.arange(L)[:, None], 5e5)
        qr = oracle.rope_rotate(b.q[r:r + 1].astype(np.float64), np.array([[L - 1]]), 5e5)
        np.testing.assert_allclose(O[r:r + 1], sdpa(qr, kr, v, b.sm_scale), rtol=0, atol=1e-12)


def test_rope_streaming_readings():
    """Streaming positions: equal to absolute when everything is visible, equal to
    absolute when there are no sinks (only relative offsets matter), different
    once sinks sit outside the window."""
    kw = dict(qo=1, causal=True, rope_theta=500000.0, seed=27, d=32)
    short = small_paged(kv=(10, 14), window=16, sink=4, rope="streaming", **kw)
    O1, L1 = oracle_attention(short)
    O2, L2 = oracle_attention(short, rope="absolute")
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    nosink = small_paged(kv=(60, 90), window=16, sink=0, rope="streaming", **kw)
    O1, L1 = oracle_attention(nosink)
    O2, L2 = oracle_attention(nosink, rope="absolute")
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    np.testing.assert_allclose(L1, L2, atol=1e-12)
    sinks = small_paged(kv=(60, 90), window=16, sink=4, rope="streaming", **kw)
    O1, _ = oracle_attention(sinks)
    O2, _ = oracle_attention(sinks, rope="absolute")
    assert np.abs(O1 - O2).max() > 1e-6


def test_rope_streaming_positions_brute_force():
    """Streaming key position = number of visible keys before it, counted by brute force."""
    L, qpos, window, sink = 50, 49, 8, 3
    vis = [j for j in range(L) if oracle.visible(qpos, np.array([j]), L, True, window, sink)[0]]
    pk, pq = oracle.key_positions(qpos, np.array(vis), "streaming")
    for j, p in zip(vis, pk):
        assert p == sum(1 for x in vis if x < j)
    assert pq == len(vis) - 1


def test_round_to_bf16_matches_torch():
    """The oracle's bf16 storage rounding equals torch's float32 -> bfloat16 conversion, on normal
    draws, wide magnitudes, subnormals, signed zeros and exact ties (both parities)."""
    import torch
    rng = np.random.default_rng(29)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e30,
                        rng.standard_normal(2000) * 1e-30, [0.0, -0.0, 1e-40, -3e-41]])
    kept = rng.integers(0, 1 << 16, size=4000, dtype=np.uint64) << 16
    ties = (kept | 0x8000) & 0x7F7FFFFF  # exactly half a bf16 unit below the next value
    x = np.concatenate([x, ties.astype(np.uint32).view(np.float32).astype(np.float64)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x)
    np.testing.assert_array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("mode", ["streaming", "absolute"])
def test_rope_stored_without_rounding_is_rope_attention(mode):
    """The rotate-store-attend reading with the identity as storage equals the RoPE attention of
    attention() (window, sinks, both position modes); bf16 storage moves it."""
    b = small_paged(kv=(70, 9, 33, 120), qo=1, causal=True, window=24, sink=3, rope=mode, rope_theta=500000.0,
                    seed=31, d=32, dtype=W.BF16)
    O1, L1 = oracle_attention(b)
    O2, L2 = oracle.attention_rope_stored(b.q, b.qo_indptr, b.kv_len, oracle_kv(b), b.num_kv_heads, b.sm_scale,
                                          b.window, b.sink, mode, b.rope_theta, store=lambda x: x)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-12)
    O3, L3 = oracle.attention_rope_stored(b.q, b.qo_indptr, b.kv_len, oracle_kv(b), b.num_kv_heads, b.sm_scale,
                                          b.window, b.sink, mode, b.rope_theta)
    assert 1e-6 < np.abs(L3 - L1).max() < 1e-1


# ---------------------------------------------------------------- plan

def _params(**kw):
    base = dict(num_qo_heads=8, num_kv_heads=2, tile_q=16, tile_kv=16, num_workers=8, split_factor=2,
                min_chunk=32, max_chunk=0, item_overhead=0, max_items_per_worker=64, max_slots=4096,
                max_merge=4096)
    base.update(kw)
    return oracle.PlanParams(**base)


def _coverage_check(qo, kv, p, plan):
    g = p.num_qo_heads // p.num_kv_heads
    # every (unit, visible key) covered exactly once
    for (r, h, row_lo, row_hi, lo, hi, sink_hi) in plan["units"]:
        mine = [it for it in plan["items"] if tuple(it[:4]) == (r, h, row_lo, row_hi)]
        cover = np.zeros(int(kv[r]), dtype=np.int64)
        for it in mine:
            cover[it[4]:it[5]] += 1
        want = np.zeros(int(kv[r]), dtype=np.int64)
        want[lo:hi] = 1
        want[0:sink_hi] += 1
        assert np.array_equal(cover, want)
        # every key visible to some row of the unit is inside [lo,hi) or the sinks
        for row in range(row_lo, row_hi):
            qpos = int(kv[r]) - int(qo[r]) + row // g
            vis = oracle.visible(qpos, np.arange(int(kv[r])), int(kv[r]), p.causal, p.window, p.sink)
            assert (want[vis] == 1).all()
    Lc = plan["chunk"]
    for it in plan["items"]:
        if not (it[4] == 0 and p.window > 0 and it[5] <= p.sink):
            lo = [u for u in plan["units"] if tuple(u[:4]) == tuple(it[:4])][0][4]
            lo_a = lo // p.tile_kv * p.tile_kv  # chunk grid: the unit's first key rounded down to tile_kv
            assert (it[4] - lo_a) % Lc == 0 or it[4] == lo
            assert it[4] % p.tile_kv == 0 or it[4] == lo
            assert it[5] - it[4] <= Lc


@pytest.mark.parametrize("causal,window,sink", [(False, 0, 0), (True, 0, 0), (True, 24, 4)])
def test_plan_coverage_and_bounds(causal, window, sink):
    rng = np.random.default_rng(3)
    kv = rng.integers(1, 300, size=9)
    qo = np.minimum(kv, rng.integers(0, 40, size=9))
    p = _params(causal=causal, window=window, sink=sink)
    plan = oracle.plan_ref(qo, kv, p)
    _coverage_check(qo, kv, p, plan)
    cost = plan["cost"]
    # LPT makespan bound
    assert plan["load"].max() <= cost.sum() / p.num_workers + cost.max()
    assert sum(len(x) for x in plan["worker_items"]) == len(plan["items"])
    # loads are consistent with the lists
    for w, lst in enumerate(plan["worker_items"]):
        assert plan["load"][w] == sum(cost[i] for i in lst)
    # slots: consecutive per multi-chunk unit, matching the merge table
    for (r, h, rlo, rhi, first, n, pfx_first, pfx_n) in plan["merge"]:
        assert pfx_first == 0 and pfx_n == 0  # no shared prefix
        its = [it for it in plan["items"] if tuple(it[:4]) == (r, h, rlo, rhi)]
        assert [it[6] for it in its] == list(range(first, first + n))


def test_plan_window_chunks_follow_the_unit_start():
    """A window unit's chunk grid starts at its first key rounded down to tile_kv: a 4096-key window
    that starts on a 16-key boundary is exactly eight 512-key chunks (plus the sink chunk), one that
    starts inside a block gets a short first chunk and a tail of fewer than 16 keys."""
    p = _params(num_qo_heads=8, num_kv_heads=1, num_workers=8, split_factor=1, min_chunk=512, max_chunk=512,
                tile_kv=16, causal=True, window=4096, sink=4)
    # query at kv_len - 1: the window starts at kv_len - 4096, i.e. at key 160 and at key 167
    plan = oracle.plan_ref([1, 1], [4096 + 160, 4096 + 167], p)
    assert plan["chunk"] == 512
    by_req = {r: [(int(a), int(b)) for (rr, _, _, _, a, b, _) in plan["items"] if rr == r] for r in (0, 1)}
    assert by_req[0] == [(160 + 512 * k, 160 + 512 * (k + 1)) for k in range(8)] + [(0, 4)]
    assert by_req[1] == [(167, 672)] + [(160 + 512 * k, 160 + 512 * (k + 1)) for k in range(1, 8)] + \
        [(4256, 4263), (0, 4)]


def test_plan_decode_chunks_carry_a_sixteenth_of_slack():
    """Rule 3 by hand: one request of 512 keys, 2 kv heads, 8 workers, split 1, so C = 1024 and an even
    share is 128 keys.  A decode-tile plan (tile_q 16) targets ceil(1024 * 17 / 128) = 136 keys, rounded
    up to 144; a 128-row plan, and a two-class plan (tile_q 128 with 16-row decode tiles), take the
    even share of 128 itself."""
    common = dict(num_workers=8, split_factor=1, min_chunk=16, tile_kv=16, causal=True)
    dec = oracle.plan_ref([1], [512], _params(tile_q=16, **common))
    assert dec["total_cost"] == 1024 and dec["chunk"] == 144
    assert [(int(a), int(b)) for (_, h, _, _, a, b, _) in dec["items"] if h == 0] == \
        [(0, 144), (144, 288), (288, 432), (432, 512)]
    for kw in (dict(tile_q=128), dict(tile_q=128, decode_tile_q=16)):
        pre = oracle.plan_ref([1], [512], _params(**kw, **common))
        assert pre["total_cost"] == 1024 and pre["chunk"] == 128
        assert [(int(a), int(b)) for (_, h, _, _, a, b, _) in pre["items"] if h == 0] == \
            [(0, 128), (128, 256), (256, 384), (384, 512)]


def test_plan_greedy_each_step_takes_least_loaded():
    kv = np.array([900, 40, 300, 1200, 7, 64])
    qo = np.ones(6, dtype=np.int64)
    p = _params(num_workers=5)
    plan = oracle.plan_ref(qo, kv, p)
    cost = plan["cost"]
    order = sorted(range(len(cost)), key=lambda i: (-cost[i], i))
    pos = {i: (w, k) for w, lst in enumerate(plan["worker_items"]) for k, i in enumerate(lst)}
    load = [0] * 5
    for i in order:
        w, _ = pos[i]
        assert load[w] == min(load) and w == min(x for x in range(5) if load[x] == min(load))
        load[w] += cost[i]


def test_plan_capacity_errors():
    with pytest.raises(oracle.PlanError) as e:
        oracle.plan_ref([1] * 40, [100] * 40, _params(num_workers=2, max_items_per_worker=4))
    assert e.value.code == "CAPACITY"
    with pytest.raises(oracle.PlanError) as e:
        oracle.plan_ref([5], [3], _params())
    assert e.value.code == "INVALID_ARG"


def test_plan_golden_tiny_decode():
    """Committed plan of the tiny fp32 decode workload (written by tests/golden/make_golden.py,
    which calls only the oracle and the input generator)."""
    with open(os.path.join(HERE, "golden", "plan_tiny_decode.json")) as f:
        gold = json.load(f)
    p = oracle.PlanParams(**gold["params"])
    plan = oracle.plan_ref(gold["qo_len"], gold["kv_len"], p)
    assert plan["chunk"] == gold["chunk"]
    assert plan["items"].tolist() == gold["items"]
    assert plan["worker_items"] == gold["worker_items"]
    assert plan["merge"][:, :6].tolist() == gold["merge"]
    assert (plan["merge"][:, 6:] == 0).all()  # no shared prefix: the prefix fields stay zero


def _prefix_params(**kw):
    base = dict(num_qo_heads=4, num_kv_heads=2, tile_q=4, tile_kv=16, num_workers=8, split_factor=2,
                min_chunk=16, max_chunk=0, item_overhead=0, max_items_per_worker=64, max_slots=4096,
                max_merge=4096, causal=True, decode_tile_q=4, shared_prefix_len=70)
    base.update(kw)
    return oracle.PlanParams(**base)


def test_plan_shared_prefix_hand_derived():
    """Composable plan with a 70-token shared prefix, worked by hand.

    g = 2; requests qo [1, 2, 1], suffix kv [20, 33, 5]: T = 4 tokens, 8 global rows, so with
    tile_q = 4 each kv head has two prefix units (rows [0,4) and [4,8)).  Suffix rows 2, 4, 2 fit
    the 4-row decode tile.  C = 4*70 + 2*(20 + 33 + 5) = 396, L_c = max(16, roundup(ceil(396/16),
    16)) = 32.  Prefix chunks [0,32) [32,64) [64,70) (pfx_n = 3); suffix chunks r0 [0,20); r1
    [0,32) [32,33); r2 [0,5).  Slots in unit order: prefix (h0,t0) 0-2, (h0,t1) 3-5, (h1,t0) 6-8,
    (h1,t1) 9-11; r0h0 12; r0h1 13; r1h0 14,15; r1h1 16,17; r2h0 18; r2h1 19.  Request 1's rows
    are global rows 2..5: rows 2,3 of prefix tile 0 and rows 0,1 of tile 1."""
    plan = oracle.plan_ref([1, 2, 1], [20, 33, 5], _prefix_params())
    assert plan["chunk"] == 32 and plan["total_cost"] == 396 and plan["num_slots"] == 20
    units = plan["units"].tolist()
    assert units[:4] == [[-1, 0, 0, 4, 0, 70, 0], [-1, 0, 4, 8, 0, 70, 0], [-1, 1, 0, 4, 0, 70, 0],
                         [-1, 1, 4, 8, 0, 70, 0]]
    assert plan["merge"].tolist() == [[0, 0, 0, 2, 12, 1, 0, 3], [0, 1, 0, 2, 13, 1, 6, 3],
                                      [1, 0, 0, 4, 14, 2, 0, 3], [1, 1, 0, 4, 16, 2, 6, 3],
                                      [2, 0, 0, 2, 18, 1, 0, 3], [2, 1, 0, 2, 19, 1, 6, 3]]
    prefix_items = [it for it in plan["items"].tolist() if it[0] == -1]
    assert [(it[1], it[2], it[4], it[5], it[6]) for it in prefix_items] == [
        (0, 0, 0, 32, 0), (0, 0, 32, 64, 1), (0, 0, 64, 70, 2), (0, 4, 0, 32, 3), (0, 4, 32, 64, 4),
        (0, 4, 64, 70, 5), (1, 0, 0, 32, 6), (1, 0, 32, 64, 7), (1, 0, 64, 70, 8), (1, 4, 0, 32, 9),
        (1, 4, 32, 64, 10), (1, 4, 64, 70, 11)]
    assert plan["item_class"].tolist().count(2) == 12
    with pytest.raises(oracle.PlanError):
        oracle.plan_ref([1], [20], _prefix_params(window=8))


@pytest.mark.parametrize("tile_q,W_", [(4, 8), (8, 3), (16, 5)])
def test_plan_shared_prefix_merge_is_flat_attention(tile_q, W_):
    """Every item of a composable plan evaluated on its own (oracle.attention_partial over the dense
    prefix or the request's pages) and merged as its merge record says, rows mapped to prefix tiles
    through their global rows, equals attention over the flat layout (prefix pages followed by the
    request's own pages).  Prefix tiles straddle requests' rows; prefix and suffix both split; one
    request's suffix is tiled by tile_q (class 0), the others are decode-class units."""
    rng = np.random.default_rng(33)
    P, Hq, Hk, d, ps = 48, 8, 2, 16, 4
    qo = np.array([1, 2, 4, 1, 3, 5])    # the last request's 20 rows exceed the 16-row decode tile
    kv = np.array([9, 30, 4, 17, 25, 12])
    suf = W.paged_batch(name="s", seed=34, kv_len=kv, qo_len=qo, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d,
                        page_size=ps, dtype=W.F32, causal=True)
    pk = rng.standard_normal((P, Hk, d)).astype(np.float32)
    pv = rng.standard_normal((P, Hk, d)).astype(np.float32)
    g = Hq // Hk
    T = int(qo.sum())
    plan = oracle.plan_ref(qo, kv, _prefix_params(num_qo_heads=Hq, num_kv_heads=Hk, tile_q=tile_q, num_workers=W_,
                                                  tile_kv=4, min_chunk=4, max_chunk=8 + 4 * (W_ % 2),
                                                  decode_tile_q=16, shared_prefix_len=P))
    assert plan["merge"][:, 5].max() >= 2 and plan["merge"][0, 7] >= 2  # both parts split
    assert set(plan["item_class"].tolist()) == {0, 1, 2}
    prefix_kv = DenseKV(pk, pv, np.array([0, P]))
    kp, vp = suf.physical_pools()
    sk = PagedKV(kp, vp, suf.kv_page_indptr, suf.kv_page_indices, ps)
    part = {}
    for (r, h, rlo, rhi, lo, hi, slot) in plan["items"].tolist():
        if r < 0:
            part[slot] = oracle.attention_partial(suf.q, np.array([0, T]), np.array([P]), prefix_kv, Hk,
                                                  suf.sm_scale, 0, h, rlo, rhi, lo, hi, causal=False)
        else:
            part[slot] = oracle.attention_partial(suf.q, suf.qo_indptr, kv, sk, Hk, suf.sm_scale, r, h, rlo, rhi,
                                                  lo, hi, causal=True)
    O = np.full((T, Hq, d), np.nan)
    L = np.full((T, Hq), np.nan)
    for (r, h, rlo, rhi, first, n, pfx_first, pfx_n) in plan["merge"].tolist():
        for rr in range(rhi - rlo):
            R = int(suf.qo_indptr[r]) * g + rlo + rr
            t, pr = R // tile_q, R % tile_q
            prefix_tile_rows = [it for it in plan["items"].tolist()
                                if it[0] < 0 and it[1] == h and it[2] <= R < it[3]]
            assert {it[6] for it in prefix_tile_rows} == set(range(pfx_first + t * pfx_n, pfx_first + (t + 1) * pfx_n))
            parts = [(part[first + c][0][rr], part[first + c][1][rr]) for c in range(n)]
            parts += [(part[pfx_first + t * pfx_n + c][0][pr], part[pfx_first + t * pfx_n + c][1][pr])
                      for c in range(pfx_n)]
            o, l = oracle.merge(parts)
            tok, qh = int(suf.qo_indptr[r]) + (rlo + rr) // g, h * g + (rlo + rr) % g
            O[tok, qh], L[tok, qh] = o, l
    # flat layout: the prefix as pages shared by every request, then the request's own pages
    flat, flat_len = oracle.flat_from_composable(pk, pv, sk, kv)
    Of, Lf = oracle.attention(suf.q, suf.qo_indptr, flat_len, flat, Hk, suf.sm_scale, causal=True)
    np.testing.assert_allclose(O, Of, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lf, rtol=0, atol=1e-12)


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(4).standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(W.round_bf16(x), ref)


def test_plan_tiny_decode_by_hand():
    """The tiny decode plan worked out by hand: C = 932 key-rows over 8 workers x split 2
    gives L_c = 64; LPT places the twelve 64-cost items first (ties to the lowest
    worker), then the 63s, the 17s and the two 2-token tails on the lightest workers."""
    p = _params(num_workers=8, split_factor=2, min_chunk=32, causal=True, max_items_per_worker=16)
    plan = oracle.plan_ref([1, 1, 1, 1], [17, 64, 130, 255], p)
    assert plan["chunk"] == 64
    spans = {(int(r), int(h)): [] for r in range(4) for h in range(2)}
    for it in plan["items"]:
        spans[(int(it[0]), int(it[1]))].append((int(it[4]), int(it[5])))
    assert spans[(2, 1)] == [(0, 64), (64, 128), (128, 130)]
    assert spans[(3, 0)] == [(0, 64), (64, 128), (128, 192), (192, 255)]
    assert spans[(0, 0)] == [(0, 17)]
    assert plan["worker_items"] == [[2, 12], [3, 14], [4, 15], [5, 16], [7, 13], [8, 17], [10, 0, 6], [11, 1, 9]]


# ------------------------------------------------------------------ append (chunked prefill)

def _append_case(seed, layout="HND"):
    rng = np.random.default_rng(seed)
    ps, Hk, d = 4, 2, 8
    P = np.array([5, 0, 8, 3])           # cached tokens before the append
    n = np.array([3, 6, 0, 9])           # new tokens
    after = P + n
    pages = (after + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(pages)])
    pool = int(indptr[-1]) + 3           # some pages belong to nobody
    perm = rng.permutation(pool)[:int(indptr[-1])]
    shape = (pool, Hk, ps, d) if layout == "HND" else (pool, ps, Hk, d)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    app = np.concatenate([[0], np.cumsum(n)])
    kn = rng.standard_normal((int(app[-1]), Hk, d)).astype(np.float32)
    vn = rng.standard_normal((int(app[-1]), Hk, d)).astype(np.float32)
    return dict(k=k, v=v, indptr=indptr, perm=perm, ps=ps, P=P, n=n, after=after, app=app, kn=kn, vn=vn,
                layout=layout)


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_append_then_gather_is_prefix_plus_new(layout):
    """Gathering the appended cache (through the separately pinned gather) gives the request's old
    prefix followed by exactly its new tokens."""
    c = _append_case(70, layout)
    k2, v2 = oracle.append_paged_kv(c["k"], c["v"], c["indptr"], c["perm"], c["ps"], c["app"], c["after"],
                                    c["kn"], c["vn"], layout=layout)
    before = PagedKV(c["k"], c["v"], c["indptr"], c["perm"], c["ps"], layout)
    after = PagedKV(k2, v2, c["indptr"], c["perm"], c["ps"], layout)
    for r in range(len(c["P"])):
        P, n = int(c["P"][r]), int(c["n"][r])
        kb, vb = oracle.gather_kv(before, r, np.arange(P))
        ka, va = oracle.gather_kv(after, r, np.arange(P + n))
        a = int(c["app"][r])
        assert np.array_equal(ka, np.concatenate([kb, c["kn"][a:a + n].astype(np.float64)]))
        assert np.array_equal(va, np.concatenate([vb, c["vn"][a:a + n].astype(np.float64)]))


def test_append_leaves_other_slots_untouched():
    c = _append_case(71)
    k2, v2 = oracle.append_paged_kv(c["k"], c["v"], c["indptr"], c["perm"], c["ps"], c["app"], c["after"],
                                    c["kn"], c["vn"])
    written = np.zeros(c["k"].shape[:1] + c["k"].shape[2:3], dtype=bool)  # [page, slot]
    for r in range(len(c["P"])):
        for pos in range(int(c["P"][r]), int(c["after"][r])):
            written[int(c["perm"][int(c["indptr"][r]) + pos // c["ps"]]), pos % c["ps"]] = True
    assert written.sum() == int(c["n"].sum())
    keep = ~written
    assert np.array_equal(k2.transpose(0, 2, 1, 3)[keep], c["k"].transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(v2.transpose(0, 2, 1, 3)[keep], c["v"].transpose(0, 2, 1, 3)[keep])


def test_append_in_two_steps_equals_one():
    """Appending a request's new tokens in two chunks (the chunked-prefill schedule) leaves the
    same cache as appending them at once."""
    c = _append_case(72)
    one = oracle.append_paged_kv(c["k"], c["v"], c["indptr"], c["perm"], c["ps"], c["app"], c["after"],
                                 c["kn"], c["vn"])
    first = c["n"] // 2
    second = c["n"] - first
    idx1 = np.concatenate([np.arange(c["app"][r], c["app"][r] + first[r]) for r in range(len(c["n"]))])
    idx2 = np.concatenate([np.arange(c["app"][r] + first[r], c["app"][r + 1]) for r in range(len(c["n"]))])
    app1 = np.concatenate([[0], np.cumsum(first)])
    app2 = np.concatenate([[0], np.cumsum(second)])
    k1, v1 = oracle.append_paged_kv(c["k"], c["v"], c["indptr"], c["perm"], c["ps"], app1, c["P"] + first,
                                    c["kn"][idx1.astype(int)], c["vn"][idx1.astype(int)])
    k2, v2 = oracle.append_paged_kv(k1, v1, c["indptr"], c["perm"], c["ps"], app2, c["after"],
                                    c["kn"][idx2.astype(int)], c["vn"][idx2.astype(int)])
    assert np.array_equal(k2, one[0]) and np.array_equal(v2, one[1])


# ------------------------------------------------------------------ two tile classes (mixed launches)

def _rows_cover_exactly_once(qo, kv, plan, g, nh):
    """Every (request, kv head, query row) belongs to exactly one unit."""
    seen = {}
    for (r, h, row_lo, row_hi, *_rest) in plan["units"]:
        for row in range(row_lo, row_hi):
            seen[(int(r), int(h), row)] = seen.get((int(r), int(h), row), 0) + 1
    want = {(r, h, row): 1 for r in range(len(qo)) if qo[r] > 0 and kv[r] > 0
            for h in range(nh) for row in range(int(qo[r]) * g)}
    assert seen == want


@pytest.mark.parametrize("causal,window,sink", [(True, 0, 0), (True, 40, 4)])
def test_mixed_plan_tiles_and_coverage(causal, window, sink):
    """Requests whose rows fit a decode tile get one decode-class unit per head; the others are
    tiled by tile_q; rows and visible keys are covered exactly once and the item classes follow
    their requests."""
    rng = np.random.default_rng(12)
    kv = rng.integers(1, 400, size=10)
    qo = np.minimum(kv, np.array([1, 3, 4, 5, 40, 1, 2, 100, 4, 9]))
    p = _params(tile_q=128, tile_kv=64, min_chunk=64, decode_tile_q=16, causal=causal, window=window, sink=sink)
    g = p.num_qo_heads // p.num_kv_heads   # 4: qo_len <= 4 fits a 16-row tile
    plan = oracle.plan_ref(qo, kv, p)
    _coverage_check(qo, kv, p, plan)
    _rows_cover_exactly_once(qo, kv, plan, g, p.num_kv_heads)
    for it, cls in zip(plan["items"], plan["item_class"]):
        r = int(it[0])
        small = int(qo[r]) * g <= 16
        assert cls == (1 if small else 0)
        assert it[3] - it[2] <= (16 if small else 128)
    # per request and head: one unit exactly when the request is decode-class
    for r in range(len(qo)):
        n_units = sum(1 for u in plan["units"] if u[0] == r and u[1] == 0)
        if qo[r] * g <= 16:
            assert n_units == 1
        else:
            assert n_units == -(-int(qo[r]) * g // 128)


def test_mixed_plan_without_decode_class_is_unchanged():
    rng = np.random.default_rng(13)
    kv = rng.integers(50, 400, size=6)
    qo = np.minimum(kv, rng.integers(5, 60, size=6))  # qo_len * g > 16 everywhere
    base = _params(tile_q=128, tile_kv=64, min_chunk=64, causal=True)
    a = oracle.plan_ref(qo, kv, base)
    b = oracle.plan_ref(qo, kv, dataclasses_replace(base, decode_tile_q=16))
    assert np.array_equal(a["items"], b["items"]) and a["worker_items"] == b["worker_items"]
    assert (b["item_class"] == 0).all()


def dataclasses_replace(p, **kw):
    import dataclasses
    return dataclasses.replace(p, **kw)
