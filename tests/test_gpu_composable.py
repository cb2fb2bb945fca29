"""GPU parity of the composable format in one launch: a dense prefix shared by every request and
each request's paged suffix planned together (shared_prefix_len), run by the mixed kernel's prefix
and suffix item classes, and merged in one pass; against the oracle's composable result and against
attention over each request's flat sequence (prefix tokens, then its suffix)."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import oracle
import workloads as W
from block_sparse_kv_plan_amd.attention import BatchAttention, tensors_for
from oracle.attention import DenseKV
from tests.gpu_util import compare, require_gpu, say
from tests.helpers import oracle_kv
from workloads.device import upload

pytestmark = pytest.mark.gpu

ONE_LAUNCH = dict(tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE)


def run_one_launch(suffix, prefix_k, prefix_v, num_workers=None, **plan_kw):
    """Plan + one run + merge of a composable batch; returns (O, LSE) as float64 arrays and the plan."""
    dev = require_gpu()
    P = prefix_k.shape[0]
    du = upload(suffix)
    pk = torch.from_numpy(prefix_k).to(torch.bfloat16).to(dev)
    pv = torch.from_numpy(prefix_v).to(torch.bfloat16).to(dev)
    attn = BatchAttention.create(device=dev, num_workers=num_workers, num_qo_heads=suffix.num_qo_heads,
                                 num_kv_heads=suffix.num_kv_heads, head_dim=suffix.head_dim, dtype=bsk.DTYPE_BF16,
                                 page_size=suffix.page_size, causal=True, max_batch=suffix.batch_size,
                                 shared_prefix_len=P, **ONE_LAUNCH, **plan_kw)
    T = int(suffix.qo_indptr[-1])
    out = torch.full((T, suffix.num_qo_heads, suffix.head_dim), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((T, suffix.num_qo_heads), float("nan"), dtype=torch.float32, device=dev)
    t = tensors_for(attn.problem, du["q"], du["k"], du["v"], out, lse, page_indices=du["pages"], prefix_k=pk,
                    prefix_v=pv)
    info = attn.plan(suffix.qo_indptr, suffix.kv_len, du["kv_indptr"])
    say(f"  one-launch plan: W={info.num_workers} items={info.num_items} chunk={info.chunk} slots={info.num_slots} "
        f"merges={info.num_merge}")
    attn.run(t)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), info


def flat_reference(suffix, prefix_k, prefix_v):
    """Attention over each request's flat sequence: the prefix tokens, then its own suffix tokens (read
    through the oracle's gather), causal, queries the sequence's last qo_len tokens."""
    P = prefix_k.shape[0]
    kv = oracle_kv(suffix)
    ks, vs, indptr = [], [], [0]
    for r in range(suffix.batch_size):
        k, v = oracle.gather_kv(kv, r, np.arange(int(suffix.kv_len[r])))
        ks += [prefix_k.astype(np.float64), k]
        vs += [prefix_v.astype(np.float64), v]
        indptr.append(indptr[-1] + P + int(suffix.kv_len[r]))
    flat = DenseKV(np.concatenate(ks), np.concatenate(vs), np.asarray(indptr))
    return oracle.attention(suffix.q, suffix.qo_indptr, suffix.kv_len.astype(np.int64) + P, flat,
                            suffix.num_kv_heads, suffix.sm_scale, causal=True)


def test_shared_prefix_one_launch_full():
    """16384-token dense prefix + 64 paged suffixes uniform [128, 1024], one query token each: the
    benchmarked one-launch plan (default workers, two target chunks per worker), every token and head
    against oracle.composable."""
    c = W.shared_prefix()
    pre, suf = c.prefix, c.suffix
    say("composable one launch: 16384-token prefix, 64 branches")
    O, L, info = run_one_launch(suf, pre.dense_k, pre.dense_v, split_factor=2)
    assert info.num_merge == 64 * 8
    ref = oracle.composable(suf.q, DenseKV(pre.dense_k, pre.dense_v, pre.kv_indptr), 16384,
                            oracle_kv(suf, physical=True), suf.kv_len, suf.num_kv_heads, suf.sm_scale)
    compare(suf, O, L, ref=ref)


@pytest.mark.parametrize("case", [
    dict(P=1000, qo=[1, 2, 4, 1, 3, 1], kv=[9, 300, 64, 1, 1000, 33], ps=16, W=24),     # prefix tail tile
    dict(P=4096, qo=[1, 40, 1, 2], kv=[500, 700, 17, 2], ps=16, W=40),                  # a 128-row suffix
    dict(P=64, qo=[1] * 70, kv=[int(x) for x in np.arange(70) * 7 + 1], ps=8, W=64),    # 280 rows: 3 tiles
    dict(P=333, qo=[3, 1, 4], kv=[3, 129, 4], ps=1, W=7),
    dict(P=2000, qo=[1, 1], kv=[100, 5000], ps=64, W=16),
])
def test_shared_prefix_one_launch_small(case):
    """Prefix lengths off the 64-key tile, global query rows whose requests straddle prefix tiles,
    decode-class and 128-row suffix units, several page sizes; prefix and suffixes split."""
    rng = np.random.default_rng(case["P"])
    Hq, Hk, d = 16, 4, 128
    suf = W.paged_batch(name=f"composable-{case['P']}", seed=case["P"] % 97, kv_len=case["kv"], qo_len=case["qo"],
                        num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d, page_size=case["ps"], dtype=W.BF16,
                        causal=True)
    pk = W.round_bf16(rng.standard_normal((case["P"], Hk, d)).astype(np.float32))
    pv = W.round_bf16(rng.standard_normal((case["P"], Hk, d)).astype(np.float32))
    say(f"composable one launch: P={case['P']} qo={case['qo'][:6]} page {case['ps']}")
    O, L, info = run_one_launch(suf, pk, pv, num_workers=case["W"], min_chunk=64, max_chunk=256,
                                tile_kv=max(64, case["ps"]))
    assert info.num_slots == info.num_items
    compare(suf, O, L, ref=flat_reference(suf, pk, pv))


def test_shared_prefix_rejects_unsupported_modes():
    dev = require_gpu()
    for kw in (dict(fused_merge=1), dict(window=64, sink=4), dict(tile_q=bsk.TILE_PREFILL_256)):
        args = dict(ONE_LAUNCH, **kw)
        with pytest.raises(bsk.BskError):
            BatchAttention.create(device=dev, num_workers=8, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                                  dtype=bsk.DTYPE_BF16, causal=True, max_batch=4, shared_prefix_len=100, **args)
