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
