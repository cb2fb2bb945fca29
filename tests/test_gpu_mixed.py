"""GPU parity of the mixed launch: decode-class (16-row) and prefill-class (128-row) items of one
batch in one persistent kernel, against the oracle, and item for item against the single-class
kernels."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import workloads as W
from tests import planbuf
from tests.gpu_util import compare, require_gpu, run, say, upload
from tests.helpers import oracle_attention_all

pytestmark = pytest.mark.gpu

MIXED = dict(tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE)


def small(seed, kv, qo, Hq=16, Hk=4, d=128, ps=16, **kw):
    return W.paged_batch(name=f"mixed-{seed}", seed=seed, kv_len=list(kv), qo_len=list(qo), num_qo_heads=Hq,
                         num_kv_heads=Hk, head_dim=d, page_size=ps, dtype=W.BF16, **kw)


def classes(attn):
    return np.concatenate(planbuf.decode(attn.int_ws.cpu().numpy())["worker_class"])


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("indep", [0, 1])
def test_mixed_small(d, fused, indep):
    """Decode rows (qo_len * g <= 16: 1-4 tokens with g = 4), prefill requests over several 128-row
    tiles with a ragged tail, empty requests; split chunks of both classes are merged."""
    qo = [1, 300, 1, 4, 0, 5, 1, 129, 2, 1]
    kv = [700, 1000, 33, 130, 9, 77, 1, 129, 1500, 2048]
    b = small(120 + d, kv, qo, d=d, causal=True)
    say(f"mixed small d={d} fused={fused} indep={indep}")
    O, L, attn, _ = run(b, num_workers=24, min_chunk=64, split_factor=2, fused_merge=fused,
                        independent_kv_strides=indep, **MIXED)
    cls = classes(attn)
    assert set(np.unique(cls)) == {0, 1} and attn.info.num_merge > 0
    compare(b, O, L)


@pytest.mark.parametrize("ps", [1, 8, 64])
def test_mixed_page_sizes(ps):
    qo = [1, 200, 3, 1, 64]
    kv = [500, 450, 97, 1, 300]
    b = small(130 + ps, kv, qo, Hq=8, Hk=2, d=128, ps=ps, causal=True)
    say(f"mixed page_size={ps}")
    O, L, _, _ = run(b, num_workers=16, min_chunk=max(64, ps), tile_kv=max(64, ps), **MIXED)
    compare(b, O, L)


def test_mixed_window_sink():
    qo = [1, 700, 1, 8, 1]
    kv = [5000, 1800, 300, 4100, 64]
    b = small(140, kv, qo, Hq=16, Hk=2, d=128, causal=True, window=1024, sink=4, poison_invisible=True)
    say("mixed window + sink")
    O, L, _, _ = run(b, num_workers=32, min_chunk=256, **MIXED)
    compare(b, O, L)


def test_mixed_items_match_single_class_kernels():
    """Without splits every item of the mixed launch is one the single-class kernels also run:
    decode-class rows equal the small-tile kernel's output bit for bit (the same item body).  The
    other rows have the large-tile kernel's LSE bit for bit; their O differs only in how the sum
    of the bf16 probabilities that divides it is formed (a ones-operand MFMA in the large-tile
    kernel, v_dot2 in the mixed launch, whose register budget is full), i.e. in the last bits."""
    qo = [1, 300, 1, 4, 1, 129, 2, 1]
    kv = [700, 1000, 33, 130, 1, 2000, 1500, 4000]
    b = small(150, kv, qo, d=128, causal=True)
    say("mixed vs single-class kernels")
    d = upload(b)
    kw = dict(num_workers=24, min_chunk=4096, split_factor=1, dev_tensors=d)
    Om, Lm, attn, _ = run(b, **MIXED, **kw)
    assert attn.info.num_merge == 0
    Od, Ld, _, _ = run(b, tile_q=bsk.TILE_DECODE, **kw)
    Op, Lp, _, _ = run(b, tile_q=bsk.TILE_PREFILL, **kw)
    small_req = np.asarray(qo) * 4 <= bsk.TILE_DECODE
    tok_small = np.repeat(small_req, qo)
    assert np.array_equal(Om[tok_small], Od[tok_small]) and np.array_equal(Lm[tok_small], Ld[tok_small])
    assert np.array_equal(Lm[~tok_small], Lp[~tok_small])
    # two fp32 sums of the same n bf16 values differ by at most about 2 n 2^-24 of the sum (n <= 4000)
    np.testing.assert_allclose(Om[~tok_small], Op[~tok_small], rtol=5e-4, atol=1e-7)
    compare(b, Om, Lm)


def test_mixed_workers_and_rejections():
    dev = require_gpu()
    p = bsk.attention.make_problem(num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype=bsk.DTYPE_BF16,
                                   num_workers=1, max_batch=8, **MIXED)
    n = bsk.device_workers(p)
    props = torch.cuda.get_device_properties(dev)
    say(f"mixed workers {n} on {props.multi_processor_count} CUs")
    assert n == 2 * props.multi_processor_count
    with pytest.raises(bsk.BskError):  # the mixed launch is built for bf16 only
        run(W.paged_batch(name="mixed-f32", seed=160, kv_len=[100, 50], qo_len=[1, 40], num_qo_heads=8,
                          num_kv_heads=2, head_dim=64, page_size=16, dtype=W.F32), **MIXED)


def test_mixed_full():
    """The benchmarked mixed batch (64 decode requests, 4 prefill chunks) with default workers and
    plan; every query token and head is compared with the oracle."""
    b = W.mixed()
    say(f"mixed full: {int(b.qo_indptr[-1])} query tokens, {b.batch_size} requests")
    O, L, attn, _ = run(b, **MIXED)
    say(f"  plan: W={attn.info.num_workers} items={attn.info.num_items} merges={attn.info.num_merge}")
    compare(b, O, L, ref=oracle_attention_all(b))
