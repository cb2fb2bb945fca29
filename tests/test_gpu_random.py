"""GPU parity on seeded random configurations: each case draws a batch (lengths, heads, head
dim, page size, KV layout, masking, RoPE, dtype) and plan settings (tile class, workers, split
factor, chunk minimum, in-kernel or separate merge, shared or independent K/V strides) from one
seeded generator, runs plan + run + merge through the C ABI and compares every output row with
the oracle.  Sizes stay small enough for the oracle to finish in about a second per case."""
import numpy as np
import pytest

import block_sparse_kv_plan_amd as bsk
import workloads as W
from tests.gpu_util import compare, run, say

pytestmark = pytest.mark.gpu

N_CASES = 64


def draw(seed):
    """(batch, plan keyword arguments, tolerances) of case `seed`."""
    rng = np.random.default_rng([2024, seed])
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    kind = pick(["decode", "decode", "prefill128", "prefill256", "mixed"])
    tile_q = {"decode": bsk.TILE_DECODE, "prefill256": bsk.TILE_PREFILL_256}.get(kind, bsk.TILE_PREFILL)
    decode = kind == "decode"
    B = int(rng.integers(1, 5))
    Hk = pick([1, 2, 4])
    g = pick([1, 2, 4, 8])
    d = pick([64, 128])
    dense = kind != "mixed" and rng.random() < 0.2
    dtype = W.F32 if (decode and rng.random() < 0.3) else W.BF16
    rope = "none"
    if decode and dtype == W.BF16 and not dense and rng.random() < 0.35:
        rope = pick(["streaming", "absolute"])
    causal = True if rope == "streaming" else bool(rng.random() < 0.8)
    window = sink = 0
    if not dense and rng.random() < 0.5:
        window = int(rng.integers(1, 600))
        sink = int(rng.integers(0, 9))
    if rope == "streaming" and window == 0 and rng.random() < 0.7:
        window, sink = int(rng.integers(1, 600)), int(rng.integers(0, 9))
    kv = rng.integers(1, 1500, size=B)
    if decode:
        qmax = 1 if rope == "streaming" else pick([1, 1, 3])
        qo = np.minimum(kv, rng.integers(1, qmax + 1, size=B))
    else:  # a mix of short (decode-class in the mixed launch) and long queries
        qo = np.minimum(kv, np.where(rng.random(B) < 0.4, rng.integers(1, 4, size=B), rng.integers(1, 161, size=B)))
    ps = pick([1, 4, 16, 16, 64])
    name = f"random-{seed}"
    if dense:
        b = W.dense_batch(name=name, seed=500 + seed, kv_len=kv, qo_len=qo, num_qo_heads=Hk * g, num_kv_heads=Hk,
                          head_dim=d, dtype=dtype, causal=causal)
    else:
        b = W.paged_batch(name=name, seed=500 + seed, kv_len=kv, qo_len=qo, num_qo_heads=Hk * g, num_kv_heads=Hk,
                          head_dim=d, page_size=ps, dtype=dtype, causal=causal, window=window, sink=sink, rope=rope,
                          rope_theta=500000.0)
    kw = dict(tile_q=tile_q, num_workers=pick([3, 8, 32, 100]), split_factor=pick([1, 2, 4]),
              min_chunk=pick([16, 64, 256, 512]), fused_merge=int(rng.random() < 0.5),
              independent_kv_strides=int(dtype == W.BF16 and rng.random() < 0.3))
    if kind == "mixed":
        kw["decode_tile_q"] = bsk.TILE_DECODE  # one launch for both tile classes
    tol = dict(o_tol=1e-4, lse_tol=1e-4) if dtype == W.F32 else {}
    return b, kw, tol


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    b, kw, tol = draw(seed)
    say(f"random case {seed}: B={b.batch_size} Hq={b.num_qo_heads} Hk={b.num_kv_heads} d={b.head_dim} "
        f"{b.kv_mode} ps={b.page_size} {b.dtype} causal={b.causal} window={b.window} sink={b.sink} "
        f"rope={b.rope} kv={list(b.kv_len)} qo={list(np.diff(b.qo_indptr))} {kw}")
    O, L, attn, _ = run(b, **kw)
    compare(b, O, L, **tol)
