"""GPU parity on degenerate and extreme inputs: very long sequences (chunks at the kernels'
page-list capacity), one-key windows, sinks beyond the window start, prefill without a cached
prefix, batches that are almost all empty."""
import numpy as np
import pytest

import block_sparse_kv_plan_amd as bsk
import workloads as W
from tests.gpu_util import compare, run, say

pytestmark = pytest.mark.gpu


def batch(seed, kv, qo=1, Hq=8, Hk=1, d=128, ps=16, **kw):
    return W.paged_batch(name=f"edge-{seed}", seed=seed, kv_len=list(kv), qo_len=qo, num_qo_heads=Hq,
                         num_kv_heads=Hk, head_dim=d, page_size=ps, dtype=W.BF16, **kw)


@pytest.mark.parametrize("ps", [16, 1])
def test_decode_long_sequence_at_chunk_capacity(ps):
    """200k keys: with max_chunk 0 the plan caps chunks at the page list the kernels stage (1024
    pages: 16384 keys at page 16, 1024 keys at page 1), so one unit becomes many chunks."""
    kv = [200000, 3] if ps == 16 else [40000, 3]
    b = batch(300 + ps, kv, ps=ps, causal=True)
    say(f"long decode ps={ps}: kv {kv}")
    O, L, attn, _ = run(b, num_workers=4, split_factor=1, min_chunk=512)
    assert attn.info.chunk == 1024 * ps  # the cap, not C / W
    assert attn.info.num_merge >= 1
    compare(b, O, L)


ALL_TILES = [bsk.TILE_DECODE, bsk.TILE_PREFILL, bsk.TILE_PREFILL_256]


@pytest.mark.parametrize("tile_q", ALL_TILES)
@pytest.mark.parametrize("window,sink", [(1, 0), (1, 3), (2, 1)])
def test_tiny_windows(tile_q, window, sink):
    """A window of one or two keys, with or without sinks: a query sees itself (and its
    predecessor), plus the first `sink` keys."""
    qo = [1, 1, 1] if tile_q == bsk.TILE_DECODE else [40, 130, 1]
    kv = [300, 5, 1] if tile_q == bsk.TILE_DECODE else [300, 130, 1]
    b = batch(310 + window * 10 + sink, kv, qo=qo, Hq=16, Hk=4, causal=True, window=window, sink=sink)
    say(f"tiny window tile_q={tile_q} window={window} sink={sink}")
    O, L, _, _ = run(b, tile_q=tile_q, num_workers=16, split_factor=2, min_chunk=64)
    compare(b, O, L)


@pytest.mark.parametrize("tile_q", ALL_TILES)
def test_sinks_past_the_window_start_and_wide_windows(tile_q):
    """sink larger than the window start (the sink range stops at the window) and windows wider
    than the sequence (no effect)."""
    qo = [1, 1, 1] if tile_q == bsk.TILE_DECODE else [64, 200, 7]
    kv = [600, 5000, 40] if tile_q == bsk.TILE_DECODE else [600, 5000, 40]
    for window, sink in ((100, 550), (10000, 4)):
        b = batch(320 + window % 97, kv, qo=qo, Hq=16, Hk=2, causal=True, window=window, sink=sink)
        say(f"window={window} sink={sink} tile_q={tile_q}")
        O, L, _, _ = run(b, tile_q=tile_q, num_workers=24, split_factor=2, min_chunk=64)
        compare(b, O, L)


def test_prefill_without_cached_prefix():
    """qo_len == kv_len: the first row of a request sees one key, rows straddle tiles and tails."""
    kv = [1, 2, 3, 127, 129, 300]
    b = batch(330, kv, qo=kv, Hq=32, Hk=8, causal=True)
    say("prefill without prefix")
    for tq in (bsk.TILE_PREFILL, bsk.TILE_PREFILL_256):
        O, L, _, _ = run(b, tile_q=tq, num_workers=32)
        compare(b, O, L)


def test_noncausal_prefill_group_of_one():
    b = batch(331, [200, 70], qo=[100, 70], Hq=4, Hk=4, d=64, causal=False)
    O, L, _, _ = run(b, tile_q=bsk.TILE_PREFILL, num_workers=8, min_chunk=64)
    compare(b, O, L)


@pytest.mark.parametrize("tile_q", ALL_TILES)
def test_almost_all_requests_empty(tile_q):
    """Nine empty requests around one real one, and a batch whose only request has one key."""
    kv = [0] * 4 + [777] + [0] * 5
    qo = [0] * 4 + [1 if tile_q == bsk.TILE_DECODE else 300] + [0] * 5
    b = batch(332, kv, qo=qo, Hq=8, Hk=2, causal=True)
    O, L, _, _ = run(b, tile_q=tile_q, num_workers=16, min_chunk=64)
    compare(b, O, L)
    b1 = batch(333, [1], qo=[1], Hq=8, Hk=2, causal=True)
    O, L, _, _ = run(b1, tile_q=tile_q, num_workers=16)
    compare(b1, O, L)


@pytest.mark.parametrize("tile_q", [bsk.TILE_PREFILL, bsk.TILE_PREFILL_256])
@pytest.mark.parametrize("indep", [0, 1])
def test_head_dim_64_window_sink_split_chunks(tile_q, indep):
    """d = 64 with a sliding window, sinks and chunks split over several workers (merged), both
    K/V stride modes; rows past the last 256-row tile's end and a key range that starts inside
    a tile."""
    kv = [700, 1500, 90, 2100]
    qo = [300, 70, 90, 513]
    b = batch(340 + indep, kv, qo=qo, Hq=16, Hk=4, d=64, ps=8, causal=True, window=333, sink=5)
    say(f"d64 window+sink tile_q={tile_q} indep={indep}")
    O, L, attn, _ = run(b, tile_q=tile_q, num_workers=40, split_factor=3, min_chunk=128, independent_kv_strides=indep)
    assert attn.info.num_merge > 0
    compare(b, O, L)


@pytest.mark.parametrize("tile_q", ALL_TILES)
def test_units_split_into_many_chunks(tile_q):
    """Units cut into 20-30 chunks of 64 keys: the merge reads the chunks of a row in groups of
    eight, so its running reference moves between groups, and with causal prefill rows the
    last chunks hold no visible key for the unit's first rows (partial LSE = -inf).  The
    in-kernel merge gives the same bits."""
    qo = [1, 1, 1] if tile_q == bsk.TILE_DECODE else [40, 130, 3]
    kv = [1500, 1100, 37] if tile_q == bsk.TILE_DECODE else [1500, 1100, 37]
    b = batch(330, kv, qo=qo, Hq=8, Hk=2, causal=True)
    say(f"many chunks tile_q={tile_q}")
    O1, L1, attn, _ = run(b, tile_q=tile_q, num_workers=8, split_factor=64, min_chunk=64, fused_merge=0)
    assert attn.info.chunk == 64 and attn.info.num_merge >= 2
    assert attn.info.num_slots >= 9 * attn.info.num_merge  # more than one group of eight per unit on average
    compare(b, O1, L1)
    O2, L2, _, _ = run(b, tile_q=tile_q, num_workers=8, split_factor=64, min_chunk=64, fused_merge=1)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
