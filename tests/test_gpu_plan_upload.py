"""The plan's upload into the int workspace: byte-identical to the host plan for a pinned host
buffer (copied by a kernel through the buffer's device address), for a pinned buffer that starts
inside a larger allocation, for pageable host memory (hipMemcpyAsync) and for a host-only plan
uploaded afterwards by bsk_upload_plan; several plans in a row on one stream.  Checked before any attention kernel reads such a plan."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import workloads as W
from block_sparse_kv_plan_amd.attention import make_problem
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


def _problem(b, W_=768):
    return make_problem(num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                        dtype=bsk.DTYPE_BF16, page_size=b.page_size, causal=True, tile_q=bsk.TILE_DECODE,
                        num_workers=W_, max_batch=b.batch_size)


def _lengths(b):
    i32 = lambda x: np.ascontiguousarray(x, dtype=np.int32)
    return i32(b.qo_indptr), i32(b.kv_len), i32(b.kv_page_indptr)


@pytest.mark.parametrize("kind", ["pinned", "pinned_offset", "pageable", "deferred"])
def test_plan_upload_is_the_host_plan(kind):
    dev = require_gpu()
    stream = torch.cuda.current_stream()
    for seed, batch in ((2, 64), (9, 7), (11, 130)):
        b = W.llama3_decode(batch=batch) if seed == 2 else W.paged_batch(
            name=f"upload-{seed}", seed=seed, kv_len=W.llama3_decode_lengths(seed=seed, batch=batch)[1], qo_len=1,
            num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=W.BF16, causal=True)
        p = _problem(b)
        int_b, _, host_b = bsk.workspace_query(p)
        say(f"plan upload {kind}: batch {batch}")
        int_ws = torch.full((int_b,), 0xAB, dtype=torch.uint8, device=dev)
        if kind in ("pinned", "deferred"):
            host = torch.empty(host_b, dtype=torch.uint8, pin_memory=True)
        elif kind == "pinned_offset":
            host = torch.empty(host_b + 4096, dtype=torch.uint8, pin_memory=True)[4096:]
        else:
            host = np.zeros(host_b, dtype=np.uint8)
        if kind == "deferred":  # host-only plan, then bsk_upload_plan
            info = bsk.plan(p, *_lengths(b), host)
            bsk.upload_plan(p, info, host, int_ws, stream)
        else:
            info = bsk.plan(p, *_lengths(b), host, int_ws, stream)
        torch.cuda.synchronize()
        used = int(info.used_bytes)
        assert 0 < used <= int_b
        want = np.asarray(host[:used]).copy() if kind == "pageable" else host[:used].numpy().copy()
        got = int_ws[:used].cpu().numpy()
        assert np.array_equal(got, want), f"first differing byte {int(np.argmax(got != want))} of {used}"
        # bytes past the plan are left alone
        assert bool((int_ws[used:used + 64] == 0xAB).all())


@pytest.mark.parametrize("next_kind", ["pinned", "pageable"])
def test_merge_states_upload_merges_and_uploads(next_kind):
    """bsk_merge_states_upload: workspace A's merge and workspace B's plan upload in one call (one
    launch for a pinned host plan, the merge then hipMemcpyAsync for pageable memory).  B's int
    workspace receives the host plan byte for byte, and A's outputs equal those of a plain
    bsk_merge_states of the same run, bit for bit."""
    from block_sparse_kv_plan_amd.attention import BatchAttention, tensors_for
    from workloads.device import upload
    dev = require_gpu()
    b = W.llama3_decode(batch=16)
    du = upload(b)
    mk = lambda: BatchAttention.create(device=dev, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                                       head_dim=b.head_dim, dtype=bsk.DTYPE_BF16, page_size=b.page_size,
                                       causal=True, max_batch=64)
    a, nxt = mk(), mk()
    T = int(b.qo_indptr[-1])
    outs = [(torch.full((T, b.num_qo_heads, b.head_dim), float("nan"), device=dev),
             torch.full((T, b.num_qo_heads), float("nan"), device=dev)) for _ in range(2)]
    stream = torch.cuda.current_stream()
    a.plan(b.qo_indptr, b.kv_len, du["kv_indptr"], stream=stream)
    assert a.info.num_merge > 0
    ts = [tensors_for(a.problem, du["q"], du["k"], du["v"], o, l, page_indices=du["pages"]) for o, l in outs]
    a.run(ts[0], stream=stream, merge=False)
    bsk.merge_states(a.problem, a.info, ts[0], a.int_ws, a.float_ws, stream)
    # the other batch's plan, built on the host only, for workspace B
    b2 = W.llama3_decode(batch=64)
    _, _, host_b = bsk.workspace_query(nxt.problem)
    host = (torch.empty(host_b, dtype=torch.uint8, pin_memory=True) if next_kind == "pinned"
            else np.zeros(host_b, dtype=np.uint8))
    info2 = bsk.plan(nxt.problem, *_lengths(b2), host)
    nxt.int_ws.fill_(0xAB)
    say(f"merge + upload, next plan in {next_kind} memory")
    bsk.merge_states_upload(a.problem, a.info, ts[1], a.int_ws, a.float_ws, nxt.problem, info2, host, nxt.int_ws,
                            stream)
    torch.cuda.synchronize()
    used = int(info2.used_bytes)
    want = np.asarray(host[:used]).copy() if next_kind == "pageable" else host[:used].numpy().copy()
    assert np.array_equal(nxt.int_ws[:used].cpu().numpy(), want)
    assert bool((nxt.int_ws[used:used + 64] == 0xAB).all())
    # ts[1] holds only the merged rows (single-chunk rows are written by the run): compare those
    rows = torch.isfinite(outs[1][1])
    assert bool(rows.any())
    assert torch.equal(outs[1][0][rows], outs[0][0][rows]) and torch.equal(outs[1][1][rows], outs[0][1][rows])
