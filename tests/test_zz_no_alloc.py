"""GPU parity of bsk_run_noalloc (run + merge with the partial states in the library's static
device scratch) against the workspace entry points (bsk_run_* + bsk_merge_states) on the same
plan, bit for bit, and against the oracle; two calls in a row, the second on a smaller batch."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import workloads as W
from block_sparse_kv_plan_amd.attention import BatchAttention, tensors_for
from tests.gpu_util import compare, require_gpu, say
from workloads.device import upload

pytestmark = pytest.mark.gpu


def _case(b, tile_q, **plan_kw):
    """(attention object planned for b, tensors, out, lse) on the default stream."""
    dev = require_gpu()
    du = upload(b)
    attn = BatchAttention.create(device=dev, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                                 head_dim=b.head_dim, dtype=bsk.DTYPE_BF16, page_size=b.page_size, causal=b.causal,
                                 tile_q=tile_q, max_batch=b.batch_size, **plan_kw)
    T = int(b.qo_indptr[-1])
    out = torch.full((T, b.num_qo_heads, b.head_dim), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((T, b.num_qo_heads), float("nan"), dtype=torch.float32, device=dev)
    t = tensors_for(attn.problem, du["q"], du["k"], du["v"], out, lse, page_indices=du["pages"])
    attn.plan(b.qo_indptr, b.kv_len, du["kv_indptr"])
    return attn, t, out, lse, du


def _both(b, tile_q, **plan_kw):
    attn, t, out, lse, du = _case(b, tile_q, **plan_kw)
    say(f"  plan: W={attn.info.num_workers} items={attn.info.num_items} slots={attn.info.num_slots} "
        f"merges={attn.info.num_merge}")
    attn.run(t)  # workspace entry points: run + merge over the float workspace
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    bsk.run_noalloc(attn.problem, attn.info, t, attn.int_ws, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), "no-alloc result differs from the workspace path"
    compare(b, out.double().cpu().numpy(), lse.double().cpu().numpy())
    return attn


@pytest.mark.parametrize("fused", [0, 1])
def test_noalloc_decode_two_calls(fused):
    big = W.llama3_decode(batch=32)
    small = W.llama3_decode(seed=12, batch=6)
    for b in (big, small):
        say(f"no-alloc decode fused={fused}: batch {b.batch_size}, {int(b.kv_len.sum())} keys")
        attn = _both(b, bsk.TILE_DECODE, split_factor=2, fused_merge=fused)
        assert attn.info.num_merge > 0


@pytest.mark.parametrize("tile_q", [bsk.TILE_PREFILL, bsk.TILE_PREFILL_256])
def test_noalloc_prefill_two_calls(tile_q):
    big = W.paged_batch(name="noalloc-prefill", seed=171, kv_len=[2000, 700, 1300, 77], qo_len=[300, 500, 300, 77],
                        num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=W.BF16, causal=True)
    small = W.paged_batch(name="noalloc-prefill-small", seed=172, kv_len=[700, 130], qo_len=[200, 129],
                          num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=W.BF16, causal=True)
    for b in (big, small):
        say(f"no-alloc prefill tile_q={tile_q}: {int(b.qo_indptr[-1])} query tokens")
        attn = _both(b, tile_q, num_workers=64, split_factor=2, min_chunk=256, max_chunk=1024)
        assert attn.info.num_merge > 0


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan with more partial-state slots than the scratch holds is refused before any launch."""
    b = W.llama3_decode()
    attn, t, out, lse, _ = _case(b, bsk.TILE_DECODE, split_factor=8, min_chunk=16, max_items_per_worker=128)
    cap = bsk.NOALLOC_SCRATCH_BYTES // (16 * (128 + 1) * 4)
    say(f"no-alloc capacity: plan slots {attn.info.num_slots}, scratch holds {cap}")
    assert attn.info.num_slots > cap
    with pytest.raises(bsk.BskError) as e:
        bsk.run_noalloc(attn.problem, attn.info, t, attn.int_ws, torch.cuda.current_stream())
    assert e.value.status == bsk.ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.isnan(out).all()  # nothing ran
