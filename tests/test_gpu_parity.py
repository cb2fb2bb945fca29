"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: max-abs(O) <= 1e-2 and max-abs(LSE) <= 1e-3 (bf16 in, fp32
accumulate); gather and plan-driven structure are bit-exact."""
import functools

import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import oracle
import workloads as W
from block_sparse_kv_plan_amd.attention import BatchAttention, merge_pair, tensors_for
from tests.gpu_util import compare, require_gpu, run, say, upload
from tests.helpers import oracle_attention_all, oracle_kv

pytestmark = pytest.mark.gpu


def small(seed, kv, qo=1, Hq=8, Hk=2, d=64, ps=16, dtype=W.BF16, **kw):
    return W.paged_batch(name=f"small-{seed}", seed=seed, kv_len=list(kv), qo_len=qo, num_qo_heads=Hq,
                         num_kv_heads=Hk, head_dim=d, page_size=ps, dtype=dtype, **kw)


# ------------------------------------------------------------------ gather

@pytest.mark.parametrize("dtype,d", [(W.F32, 64), (W.BF16, 128)])
def test_gather_bit_exact(dtype, d):
    dev = require_gpu()
    b = small(31, [17, 64, 130, 255, 1], Hq=8, Hk=2, d=d, ps=16, dtype=dtype, pool_pages=80)
    say(f"gather {dtype} d={d}")
    du = upload(b)
    attn = BatchAttention.create(device=dev, num_workers=7, num_qo_heads=8, num_kv_heads=2, head_dim=d,
                                 dtype=bsk.DTYPE_BF16 if dtype == W.BF16 else bsk.DTYPE_F32, causal=True,
                                 max_batch=8, min_chunk=32, tile_kv=16)
    info = attn.plan(b.qo_indptr, b.kv_len, du["kv_indptr"])
    from tests import planbuf
    plan = planbuf.decode(attn.host_ws.numpy())
    items = sorted((int(x[7]), x) for lst in plan["worker_items"] for x in lst)
    lens = np.array([int(x[5] - x[4]) for _, x in items])
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    n = int(lens.sum())
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    ko = torch.zeros((n, d), dtype=tdt, device=dev)
    vo = torch.zeros((n, d), dtype=tdt, device=dev)
    out = torch.empty((5, 8, d), dtype=torch.float32, device=dev)
    lse = torch.empty((5, 8), dtype=torch.float32, device=dev)
    t = tensors_for(attn.problem, du["q"], du["k"], du["v"], out, lse, page_indices=du["pages"])
    bsk.debug_gather(attn.problem, info, t, attn.int_ws, torch.from_numpy(offs).to(dev), ko, vo,
                     torch.cuda.current_stream())
    torch.cuda.synchronize()
    kp, vp = b.physical_pools()
    got_k, got_v = ko.float().cpu().numpy(), vo.float().cpu().numpy()
    for (iid, x), off, ln in zip(items, offs, lens):
        r, h, lo, hi = int(x[0]), int(x[1]), int(x[4]), int(x[5])
        tok = np.arange(lo, hi)
        pages = b.kv_page_indices[b.kv_page_indptr[r] + tok // 16]
        np.testing.assert_array_equal(got_k[off:off + ln], kp[pages, h, tok % 16, :])
        np.testing.assert_array_equal(got_v[off:off + ln], vp[pages, h, tok % 16, :])


# ------------------------------------------------------------------ decode (16-row tiles)

def test_tiny_decode_f32():
    """4 requests, kv {17,64,130,255}, 64-page permuted pool, 8/2 heads, d 64, fp32."""
    b = W.tiny_decode_f32()
    O, L, attn, _ = run(b, num_workers=8, split_factor=2, min_chunk=32)
    assert attn.info.num_merge > 0
    compare(b, O, L, o_tol=1e-5, lse_tol=1e-5)


def test_tiny_decode_f32_nhd_layout():
    b = W.tiny_decode_f32()
    O, L, _, _ = run(b, layout="NHD", num_workers=5, split_factor=3, min_chunk=16)
    compare(b, O, L, o_tol=1e-5, lse_tol=1e-5)


@pytest.mark.parametrize("split", [1, 2])
def test_llama3_decode_full(split):
    """64 requests, kv lognormal [512, 8192], 32/8 heads, d 128, bf16, page 16: the benchmarked launch
    (split factor 1, the decode default) and the finer split with more merged units."""
    b = W.llama3_decode()
    say(f"llama3 decode: {int(b.kv_len.sum())} keys, split factor {split}")
    O, L, attn, _ = run(b, split_factor=split)
    say(f"  plan: W={attn.info.num_workers} items={attn.info.num_items} chunk={attn.info.chunk} "
        f"merges={attn.info.num_merge}")
    compare(b, O, L)


def test_llama3_decode_bf16_out():
    b = W.llama3_decode(batch=16)
    O, L, _, _ = run(b, out_dtype=bsk.DTYPE_BF16)
    compare(b, O, L, out_bf16=True)


@pytest.mark.parametrize("tile_q,extra", [(bsk.TILE_PREFILL, {}), (bsk.TILE_PREFILL_256, {}),
                                          (bsk.TILE_PREFILL, dict(decode_tile_q=bsk.TILE_DECODE)),
                                          (bsk.TILE_DECODE, {})])
def test_bf16_output_few_key_rows(tile_q, extra):
    """bf16 output from every epilogue (prefill, mixed, decode; direct rows and the merge of split
    units): causal rows without cache see one, two, three ... keys, so |O| is not averaged down and
    bf16's own rounding (up to 2^-8 |O|) is part of the bound."""
    kv = [300, 77, 2, 1, 160] if tile_q != bsk.TILE_DECODE else [300, 77, 2, 1, 1600]
    qo = kv if tile_q != bsk.TILE_DECODE else [1, 1, 1, 1, 1]
    b = small(74, kv, qo=qo, Hq=8, Hk=2, d=128, causal=True)
    O, L, attn, _ = run(b, tile_q=tile_q, out_dtype=bsk.DTYPE_BF16, num_workers=8, split_factor=4, min_chunk=64,
                        **extra)
    assert attn.info.num_merge > 0  # some rows come out of the merge
    compare(b, O, L, out_bf16=True)


@pytest.mark.parametrize("case", [
    dict(d=128, ps=16, Hq=32, Hk=8, kv=[1, 15, 16, 17, 300, 1000]),
    dict(d=64, ps=1, Hq=4, Hk=4, kv=[3, 40, 77]),
    dict(d=128, ps=8, Hq=16, Hk=1, kv=[129, 64]),
    dict(d=128, ps=32, Hq=8, Hk=1, kv=[500, 33]),
    dict(d=64, ps=16, Hq=32, Hk=2, kv=[90, 260]),          # g = 16
    dict(d=128, ps=16, Hq=64, Hk=2, kv=[90, 260]),         # g = 32: a token spans two tiles
])
def test_decode_shapes(case):
    kw = dict(case)
    kv = kw.pop("kv")
    b = small(40 + kw["ps"], kv, causal=True, **kw)
    for W_, sf in [(3, 4), (64, 1)]:
        O, L, _, _ = run(b, num_workers=W_, split_factor=sf, min_chunk=16)
        compare(b, O, L)


def test_decode_multi_token_causal_and_empty_requests():
    kv = np.array([0, 50, 33, 7, 120])
    qo = np.array([0, 3, 0, 7, 5])
    b = small(50, kv, qo=qo, Hq=8, Hk=2, d=128, causal=True)
    O, L, _, _ = run(b, num_workers=4, split_factor=2, min_chunk=16)
    compare(b, O, L)


def test_decode_window_sink_no_rope():
    b = small(51, [4000, 30, 700], Hq=16, Hk=2, d=128, causal=True, window=256, sink=4, poison_invisible=True)
    O, L, attn, _ = run(b, num_workers=16, split_factor=2, min_chunk=64)
    compare(b, O, L)


def test_decode_dense_kv():
    b = W.dense_batch(name="dense-decode", seed=52, kv_len=[70, 300, 1], qo_len=[1, 1, 1], num_qo_heads=8,
                      num_kv_heads=2, head_dim=128, dtype=W.BF16, causal=True)
    O, L, _, _ = run(b, num_workers=6, min_chunk=32)
    compare(b, O, L)


def test_partial_states_match_oracle_items():
    """Each split item's partial (O_c, LSE_c) in the float workspace against the oracle's
    restricted attention on the item's rows and key range."""
    b = small(53, [300, 90], Hq=8, Hk=2, d=128, causal=True)
    O, L, attn, _ = run(b, num_workers=4, split_factor=4, min_chunk=32)
    from tests import planbuf
    plan = planbuf.decode(attn.host_ws.numpy())
    fw = attn.float_ws.view(torch.float32).cpu().numpy()
    max_slots, tq, d = attn.problem.max_slots, 16, 128
    po = fw[:max_slots * tq * d].reshape(max_slots, tq, d)
    pl = fw[max_slots * tq * d:max_slots * tq * (d + 1)].reshape(max_slots, tq)
    kv = oracle_kv(b)
    checked = 0
    for lst in plan["worker_items"]:
        for x in lst:
            r, h, rlo, rhi, lo, hi, slot = (int(v) for v in x[:7])
            if slot < 0:
                continue
            ro, rl = oracle.attention_partial(b.q, b.qo_indptr, b.kv_len, kv, b.num_kv_heads, b.sm_scale, r, h,
                                              rlo, rhi, lo, hi, causal=True)
            n = rhi - rlo
            assert np.abs(po[slot, :n] - ro).max() <= 1e-2
            assert np.abs(pl[slot, :n] - rl).max() <= 1e-3
            checked += 1
    assert checked > 0


def test_determinism_and_page_permutation():
    """Two runs are bit-identical, and so are runs on two page-pool permutations of the
    same logical cache (the plan depends only on lengths)."""
    b1 = small(54, [700, 45, 1300], Hq=32, Hk=8, d=128, pool_pages=200, perm_seed=1, causal=True)
    b2 = small(54, [700, 45, 1300], Hq=32, Hk=8, d=128, pool_pages=200, perm_seed=2, causal=True)
    O1, L1, _, _ = run(b1, num_workers=32)
    O1b, L1b, _, _ = run(b1, num_workers=32)
    O2, L2, _, _ = run(b2, num_workers=32)
    assert np.array_equal(O1, O1b) and np.array_equal(L1, L1b)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    compare(b1, O1, L1)


@pytest.mark.parametrize("tile_q", [bsk.TILE_DECODE, bsk.TILE_PREFILL, bsk.TILE_PREFILL_256])
def test_fused_merge_matches_separate_merge(tile_q):
    """In-kernel merge by the last chunk of each split unit gives exactly the
    separate merge kernel's result, leaves the arrival counters at zero, and a
    second run on the same plan (no re-plan) reproduces it."""
    from tests import planbuf
    kv = np.array([900, 2000, 33, 512])
    qo = np.array([1, 1, 1, 1]) if tile_q == bsk.TILE_DECODE else np.array([100, 300, 33, 200])
    b = small(90, kv, qo=qo, Hq=32, Hk=8, d=128, causal=True)
    kw = dict(tile_q=tile_q, num_workers=32, split_factor=4, min_chunk=64)
    O1, L1, _, _ = run(b, fused_merge=0, **kw)
    O2, L2, attn, (t, out, lse, _, _) = run(b, fused_merge=1, **kw)
    assert attn.info.num_merge > 0
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    compare(b, O2, L2)
    arrivals = planbuf.decode(attn.int_ws.cpu().numpy())["arrivals"]
    assert len(arrivals) == attn.info.num_merge and (arrivals == 0).all()
    out.fill_(float("nan"))
    attn.run(t)
    torch.cuda.synchronize()
    assert np.array_equal(out.double().cpu().numpy(), O2) and np.array_equal(lse.double().cpu().numpy(), L2)


# ------------------------------------------------------------------ prefill (128- and 256-row tiles)

PREFILL_TILES = [bsk.TILE_PREFILL, bsk.TILE_PREFILL_256]


@pytest.mark.parametrize("tile_q", PREFILL_TILES)
def test_prefill_small_several_tiles(tile_q):
    kv = np.array([300, 129, 77, 1000])
    qo = np.array([300, 40, 77, 130])
    b = small(60, kv, qo=qo, Hq=8, Hk=2, d=128, causal=True)
    for W_ in (5, 64):
        say(f"prefill tile_q={tile_q} W={W_}")
        O, L, _, _ = run(b, tile_q=tile_q, num_workers=W_, split_factor=2, min_chunk=64)
        compare(b, O, L)


@pytest.mark.parametrize("tile_q", PREFILL_TILES)
def test_prefill_head_dim_64_noncausal_and_window(tile_q):
    kv = np.array([257, 64])
    b = small(61, kv, qo=np.array([100, 64]), Hq=4, Hk=4, d=64, causal=False)
    O, L, _, _ = run(b, tile_q=tile_q, num_workers=9, min_chunk=64)
    compare(b, O, L)
    b2 = small(62, kv, qo=np.array([100, 64]), Hq=8, Hk=2, d=128, causal=True, window=50, sink=3)
    O, L, _, _ = run(b2, tile_q=tile_q, num_workers=9, min_chunk=64)
    compare(b2, O, L)


@pytest.mark.parametrize("tile_q", PREFILL_TILES)
@pytest.mark.parametrize("ps,d", [(1, 128), (8, 64), (32, 128), (64, 128), (128, 128), (256, 64)])
def test_prefill_page_sizes(tile_q, ps, d):
    """Page sizes below, at and above the 64-key tile: the per-tile page slot / in-page offset
    arithmetic of full tiles and the clamped ragged tail."""
    kv = np.array([700, 64, 333, 1])
    qo = np.array([200, 64, 333, 1])
    b = small(63 + ps, kv, qo=qo, Hq=8, Hk=2, d=d, ps=ps, causal=True)
    say(f"prefill tile_q={tile_q} page_size={ps} d={d}")
    O, L, _, _ = run(b, tile_q=tile_q, num_workers=11, min_chunk=max(64, ps), tile_kv=max(64, ps))
    compare(b, O, L)


@functools.lru_cache(maxsize=1)
def ragged_prefill_reference():
    """The oracle on every query token of the ragged prefill workload (computed once per module)."""
    b = W.ragged_prefill()
    say(f"oracle: all {int(b.qo_indptr[-1])} query tokens of the ragged prefill")
    return oracle_attention_all(b)


@pytest.mark.parametrize("tile_q", PREFILL_TILES)
def test_ragged_prefill_full(tile_q):
    """16 requests, new lengths lognormal [128, 4096] appended after [0, 2048] cached keys, the
    benchmarked launch (default workers and plan); every query token and head is compared."""
    b = W.ragged_prefill()
    say(f"ragged prefill tile_q={tile_q}: {int(b.qo_indptr[-1])} query tokens")
    O, L, attn, _ = run(b, tile_q=tile_q)
    say(f"  plan: W={attn.info.num_workers} items={attn.info.num_items} chunk={attn.info.chunk} "
        f"merges={attn.info.num_merge}")
    compare(b, O, L, ref=ragged_prefill_reference())


# ------------------------------------------------------------------ composable (dense prefix + paged suffix)

def run_composable(c, prefix_workers=None, suffix_workers=None, prefix_tile=bsk.TILE_PREFILL):
    dev = require_gpu()
    pre, suf = c.prefix, c.suffix
    Op, Lp, _, _ = run(pre, tile_q=prefix_tile, num_workers=prefix_workers)
    Os, Ls, _, _ = run(suf, num_workers=suffix_workers)
    T, Hq, d = suf.q.shape
    oa = torch.from_numpy(Op.astype(np.float32)).to(dev)
    la = torch.from_numpy(Lp.astype(np.float32)).to(dev)
    ob = torch.from_numpy(Os.astype(np.float32)).to(dev)
    lb = torch.from_numpy(Ls.astype(np.float32)).to(dev)
    oo = torch.empty_like(oa)
    lo = torch.empty_like(la)
    merge_pair(oa, la, ob, lb, oo, lo)
    torch.cuda.synchronize()
    return oo.double().cpu().numpy(), lo.double().cpu().numpy()


@pytest.mark.parametrize("prefix_tile", PREFILL_TILES)
def test_shared_prefix_composable_full(prefix_tile):
    """16384-token dense prefix + 64 paged suffixes [128, 1024], merged by LSE."""
    c = W.shared_prefix()
    say(f"composable prefix tile_q={prefix_tile}")
    O, L = run_composable(c, prefix_tile=prefix_tile)
    pre, suf = c.prefix, c.suffix
    from oracle.attention import DenseKV
    kp, vp = suf.physical_pools()
    ref = oracle.composable(suf.q, DenseKV(pre.dense_k, pre.dense_v, pre.kv_indptr), 16384,
                            oracle_kv(suf, physical=True), suf.kv_len, suf.num_kv_heads, suf.sm_scale)
    compare(suf, O, L, ref=ref)


def test_composable_concurrent_matches_sequential():
    """run_composable with the suffix on a side stream (each part planned for half the GPU) gives
    the same bits as the sequential order, and the oracle's composable result."""
    dev = require_gpu()
    c = W.shared_prefix()
    pre, suf = c.prefix, c.suffix
    say("composable: concurrent vs sequential")
    from block_sparse_kv_plan_amd.attention import run_composable
    parts = []
    for bb, tq in ((pre, bsk.TILE_PREFILL), (suf, bsk.TILE_DECODE)):
        _, _, attn, (t, o, l, d, _) = run(bb, tile_q=tq, num_workers=256)
        parts.append((attn, t, (o, l)))
    outs = []
    for side in (None, torch.cuda.Stream()):
        fo = torch.full((64, 32, 128), float("nan"), dtype=torch.float32, device=dev)
        fl = torch.full((64, 32), float("nan"), dtype=torch.float32, device=dev)
        for i in range(3):  # repeated runs reuse the same plans
            run_composable(parts[0][0], parts[0][1], parts[0][2], parts[1][0], parts[1][1], parts[1][2], fo, fl,
                           side_stream=side)
        torch.cuda.synchronize()
        outs.append((fo.double().cpu().numpy(), fl.double().cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    from oracle.attention import DenseKV
    ref = oracle.composable(suf.q, DenseKV(pre.dense_k, pre.dense_v, pre.kv_indptr), 16384,
                            oracle_kv(suf, physical=True), suf.kv_len, suf.num_kv_heads, suf.sm_scale)
    compare(suf, outs[1][0], outs[1][1], ref=ref)


# ------------------------------------------------------------------ fused RoPE + window + sinks

@pytest.mark.parametrize("split", [1, 2])
def test_streaming_rope_full(split):
    """batch 8, kv uniform [32768, 131072], 64/8 heads, window 4096 + 4 sinks, RoPE theta 5e5; split
    factor 2 is the benchmarked launch (512-key chunks), 1 the decode default (528-key chunks)."""
    b = W.streaming_rope_decode()
    say(f"streaming rope: kv {b.kv_len.tolist()}, split factor {split}")
    O, L, _, _ = run(b, split_factor=split)
    compare(b, O, L)


@pytest.mark.parametrize("mode", ["streaming", "absolute"])
def test_rope_small(mode):
    b = small(70, [5000, 40, 4101, 4099], Hq=16, Hk=2, d=128, causal=True, window=4096, sink=4, rope=mode,
              rope_theta=500000.0, poison_invisible=True)
    O, L, _, _ = run(b, num_workers=24)
    compare(b, O, L)


def test_rope_head_dim_64():
    b = small(71, [900, 20], Hq=8, Hk=1, d=64, causal=True, window=128, sink=2, rope="streaming",
              rope_theta=10000.0, poison_invisible=True)
    O, L, _, _ = run(b, num_workers=6)
    compare(b, O, L)


@pytest.mark.parametrize("mode", ["absolute", "streaming"])
def test_rope_long_items(mode):
    """Items of the kernels' longest chunk (1024 pages = 16,384 keys): each wave then steps its
    (cos, sin) pairs 256 times by the 64-position rotation, the longest the recurrence runs."""
    b = small(75, [60000, 33000], Hq=8, Hk=1, d=128, causal=True, window=50000 if mode == "streaming" else 0,
              sink=4 if mode == "streaming" else 0, rope=mode, rope_theta=500000.0, poison_invisible=True)
    O, L, attn, _ = run(b, num_workers=4)
    assert attn.info.chunk == 16384
    compare(b, O, L)


@pytest.mark.parametrize("mode,window,d", [("absolute", 1, 128), ("absolute", 1, 64), ("absolute", 2, 128),
                                           ("streaming", 3, 64)])
def test_rope_rows_led_by_one_key(mode, window, d):
    """Rows that see one to three keys: the LSE is then (nearly) one rotated logit, so every bit of
    the logit's rounding reaches it.  64 requests x 64 heads, kv uniform [64, 6000]; with the
    rotated q and K rounded once to fp16 the worst row was 1.36e-3 off (window 1, absolute)."""
    rng = np.random.default_rng(72)
    kv = rng.integers(64, 6001, size=64)
    b = W.paged_batch(name=f"rope-{mode}-w{window}-d{d}", seed=73 + window + d, kv_len=kv,
                      qo_len=np.ones(64, dtype=np.int64), num_qo_heads=64, num_kv_heads=8, head_dim=d, page_size=16,
                      dtype=W.BF16, causal=True, window=window, sink=0, rope=mode, rope_theta=500000.0,
                      poison_invisible=True)
    O, L, _, _ = run(b)
    compare(b, O, L)


# ------------------------------------------------------------------ plan upload on a copy stream

@pytest.mark.parametrize("fused", [0, 1])
def test_copy_stream_uploads_alternating_plans(fused):
    """Two plan workspaces used alternately, a different batch (lengths, hence plan) every step,
    each plan uploaded on a side stream while the main stream still runs earlier steps, and the
    merges on a third stream (or merged in the kernel): every step's output equals the same step
    run in one stream, bit for bit, and the oracle.  The main stream is kept busy first, so every
    plan is made while the runs before it are still queued: a plan that did not wait for the last
    run reading its workspace would overwrite that run's plan."""
    dev = require_gpu()
    Hq, Hk, d = 32, 8, 128
    rng = np.random.default_rng(83)
    batches = [small(83 + i, rng.integers(1, 3000, size=int(rng.integers(3, 12))), Hq=Hq, Hk=Hk, d=d, causal=True)
               for i in range(6)]
    say(f"copy-stream plan uploads over 6 steps, fused merge {fused}")
    attn = [BatchAttention.create(device=dev, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d, dtype=bsk.DTYPE_BF16,
                                  causal=True, max_batch=16, fused_merge=fused) for _ in range(2)]
    busy = torch.randn((4096, 4096), dtype=torch.float32, device=dev)
    dus = [upload(bb) for bb in batches]
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def outputs():
        return [(torch.full((int(bb.qo_indptr[-1]), Hq, d), float("nan"), dtype=torch.float32, device=dev),
                 torch.full((int(bb.qo_indptr[-1]), Hq), float("nan"), dtype=torch.float32, device=dev))
                for bb in batches]

    merge_side = torch.cuda.Stream()
    results = []
    # in-stream; uploads on a copy stream; uploads and merges each on a stream of their own
    for copy_stream, merge_stream in ((None, None), (side, None), (side, merge_side)):
        outs = outputs()
        torch.cuda.synchronize()
        for _ in range(8):  # ~10 ms of queued work ahead of the first run
            busy = busy @ busy * (1.0 / 64.0)
        for i, (bb, du) in enumerate(zip(batches, dus)):
            a = attn[i % 2]
            t = tensors_for(a.problem, du["q"], du["k"], du["v"], outs[i][0], outs[i][1], page_indices=du["pages"])
            a.plan(bb.qo_indptr, bb.kv_len, du["kv_indptr"], stream=main, copy_stream=copy_stream)
            if merge_stream is None:
                a.run(t, stream=main)
            else:
                a.run(t, stream=main, merge=False)
                done = torch.cuda.Event()
                done.record(main)
                merge_stream.wait_event(done)
                a.merge(t, merge_stream)
        torch.cuda.synchronize()
        results.append([(o.double().cpu().numpy(), l.double().cpu().numpy()) for o, l in outs])
    for i, bb in enumerate(batches):
        for r in results[1:]:
            assert np.array_equal(results[0][i][0], r[i][0]) and np.array_equal(results[0][i][1], r[i][1])
        compare(bb, results[2][i][0], results[2][i][1])


@pytest.mark.parametrize("fused", [0, 1])
def test_deferred_uploads_ride_on_merges(fused):
    """Two workspaces in turn, a different batch every step, each plan's upload deferred and made
    in the same launch as the other workspace's merge of the previous step (bsk_merge_states_upload;
    with the in-kernel merge, bsk_upload_plan beside it), behind queued work: every step's output
    equals the same step with plain in-stream uploads, bit for bit, and the oracle."""
    dev = require_gpu()
    Hq, Hk, d = 32, 8, 128
    rng = np.random.default_rng(84)
    batches = [small(84 + i, rng.integers(1, 3000, size=int(rng.integers(3, 12))), Hq=Hq, Hk=Hk, d=d, causal=True)
               for i in range(6)]
    say(f"deferred uploads over 6 steps, fused merge {fused}")
    attn = [BatchAttention.create(device=dev, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d, dtype=bsk.DTYPE_BF16,
                                  causal=True, max_batch=16, fused_merge=fused) for _ in range(2)]
    dus = [upload(bb) for bb in batches]
    main = torch.cuda.current_stream()
    busy = torch.randn((4096, 4096), dtype=torch.float32, device=dev)
    results = []
    for deferred in (False, True):
        outs = [(torch.full((int(bb.qo_indptr[-1]), Hq, d), float("nan"), dtype=torch.float32, device=dev),
                 torch.full((int(bb.qo_indptr[-1]), Hq), float("nan"), dtype=torch.float32, device=dev))
                for bb in batches]
        torch.cuda.synchronize()
        for _ in range(8):
            busy = busy @ busy * (1.0 / 64.0)
        prev = None
        for i, (bb, du) in enumerate(zip(batches, dus)):
            a = attn[i % 2]
            t = tensors_for(a.problem, du["q"], du["k"], du["v"], outs[i][0], outs[i][1], page_indices=du["pages"])
            if not deferred:
                a.plan(bb.qo_indptr, bb.kv_len, du["kv_indptr"], stream=main)
                a.run(t, stream=main)
                continue
            a.plan(bb.qo_indptr, bb.kv_len, du["kv_indptr"], stream=main, defer_upload=True)
            if prev is None:
                a.upload(main)
            else:
                prev[0].merge(prev[1], main, upload_next=a)
            a.run(t, stream=main, merge=False)
            prev = (a, t)
        if prev is not None:
            prev[0].merge(prev[1], main)
        torch.cuda.synchronize()
        results.append([(o.double().cpu().numpy(), l.double().cpu().numpy()) for o, l in outs])
    for i, bb in enumerate(batches):
        assert np.array_equal(results[0][i][0], results[1][i][0]) and np.array_equal(results[0][i][1], results[1][i][1])
        compare(bb, results[1][i][0], results[1][i][1])


# ------------------------------------------------------------------ graph capture

def test_graph_capture_replan_replay():
    """run + merge captured once in a graph; new plans (different lengths) uploaded into the
    same workspace; each replay matches the oracle, with eager work between replays."""
    dev = require_gpu()
    b = small(80, [900, 2000, 33, 512], Hq=32, Hk=8, d=128, causal=True, pool_pages=400)
    du = upload(b)
    attn = BatchAttention.create(device=dev, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                                 dtype=bsk.DTYPE_BF16, causal=True, max_batch=4)
    out = torch.zeros((4, 32, 128), dtype=torch.float32, device=dev)
    lse = torch.zeros((4, 32), dtype=torch.float32, device=dev)
    t = tensors_for(attn.problem, du["q"], du["k"], du["v"], out, lse, page_indices=du["pages"])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        attn.plan(b.qo_indptr, b.kv_len, du["kv_indptr"], stream=s)
        attn.run(t, stream=s)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        attn.run(t, stream=s)
    for trial, lens in enumerate([[900, 2000, 33, 512], [17, 1500, 33, 2], [640, 640, 640, 640]]):
        kv = np.minimum(np.asarray(lens), b.kv_len)
        attn.plan(b.qo_indptr, kv, du["kv_indptr"], stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        bt = small(80, [900, 2000, 33, 512], Hq=32, Hk=8, d=128, causal=True, pool_pages=400)
        bt.kv_len = kv.astype(np.int32)
        compare(bt, out.double().cpu().numpy(), lse.double().cpu().numpy())
        _ = (out * 2).sum().item()  # eager work between replays


def test_capture_replay_alternating_workspaces():
    """BatchAttention.capture / replay as the benchmark uses them: two workspaces, a graph per
    (workspace, output) pair captured once, a new plan (other lengths) uploaded on a copy stream
    before every replay.  Every replay equals the eager run + merge of the same plan bit for bit,
    and the oracle; eager work and synchronisations run between the replays."""
    dev = require_gpu()
    lens = [[900, 2000, 33, 512], [17, 1500, 33, 2], [640, 640, 640, 640], [4000, 1, 77, 1999]]
    b = small(81, [4000, 2000, 640, 1999], Hq=32, Hk=8, d=128, causal=True)
    du = upload(b)
    attn = [BatchAttention.create(device=dev, num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype=bsk.DTYPE_BF16,
                                  causal=True, max_batch=4, split_factor=3, min_chunk=64) for _ in range(2)]
    outs = [(torch.zeros((4, 32, 128), dtype=torch.float32, device=dev), torch.zeros((4, 32), device=dev))
            for _ in range(2)]
    ts = [tensors_for(attn[0].problem, du["q"], du["k"], du["v"], o, l, page_indices=du["pages"]) for o, l in outs]
    main = torch.cuda.current_stream()
    for a in attn:
        a.plan(b.qo_indptr, b.kv_len, du["kv_indptr"], stream=main)
    torch.cuda.synchronize()
    graphs = [attn[w].capture(ts[w]) for w in range(2)]
    copy = torch.cuda.Stream()
    for step in range(8):
        w = step % 2
        kv = np.minimum(np.asarray(lens[step % 4]), b.kv_len)
        say(f"replay step {step}: workspace {w}, kv {kv.tolist()}")
        info = attn[w].plan(b.qo_indptr, kv, du["kv_indptr"], stream=main, copy_stream=copy)
        outs[w][0].fill_(float("nan"))
        attn[w].replay(graphs[w], main)
        torch.cuda.synchronize()
        got = (outs[w][0].clone(), outs[w][1].clone())
        outs[w][0].fill_(float("nan"))
        attn[w].run(ts[w], stream=main)
        torch.cuda.synchronize()
        assert torch.equal(got[0], outs[w][0]) and torch.equal(got[1], outs[w][1]), f"step {step}"
        if step < 4:
            assert info.num_merge > 0
            bt = small(81, [4000, 2000, 640, 1999], Hq=32, Hk=8, d=128, causal=True)
            bt.kv_len = kv.astype(np.int32)
            compare(bt, got[0].double().cpu().numpy(), got[1].double().cpu().numpy())
        _ = (outs[1 - w][0] * 2).sum().item()  # eager work between replays


# ------------------------------------------------------------------ K/V stride specialisation

@pytest.mark.parametrize("tile_q", [bsk.TILE_DECODE, bsk.TILE_PREFILL, bsk.TILE_PREFILL_256])
def test_kv_stride_specialisation_is_bit_identical(tile_q):
    """With equal K/V strides the shared-address kernels and the independent-stride kernels
    compute exactly the same result (only the addressing differs)."""
    kv = np.array([300, 129, 77, 1000])
    qo = np.array([1, 1, 1, 1]) if tile_q == bsk.TILE_DECODE else np.array([300, 40, 77, 130])
    b = small(97, kv, qo=qo, Hq=16, Hk=4, d=128, causal=True)
    say(f"kv stride specialisation tile_q={tile_q}")
    O1, L1, _, _ = run(b, tile_q=tile_q, num_workers=24, min_chunk=64, independent_kv_strides=0)
    O2, L2, _, _ = run(b, tile_q=tile_q, num_workers=24, min_chunk=64, independent_kv_strides=1)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    compare(b, O1, L1)


@pytest.mark.parametrize("tile_q", [bsk.TILE_DECODE, bsk.TILE_PREFILL])
def test_independent_v_strides(tile_q):
    """V in a pool with padded rows (its own strides) goes through the independent-stride kernels."""
    kv = np.array([300, 129, 77, 1000])
    qo = np.array([1, 1, 1, 1]) if tile_q == bsk.TILE_DECODE else np.array([300, 40, 77, 130])
    b = small(98, kv, qo=qo, Hq=16, Hk=4, d=128, causal=True)
    d = upload(b)
    v = d["v"]
    vpad = torch.full(v.shape[:-1] + (v.shape[-1] + 16,), float("nan"), dtype=v.dtype, device=v.device)
    vpad[..., :v.shape[-1]] = v
    d["v"] = vpad[..., :v.shape[-1]]
    assert d["v"].stride() != d["k"].stride()
    say(f"independent V strides tile_q={tile_q}")
    O, L, _, _ = run(b, tile_q=tile_q, num_workers=24, min_chunk=64, dev_tensors=d)
    compare(b, O, L)
