"""bench.py on the CPU: the one-GPU guard, and the algorithmic byte and flop counts that the
roofline fractions divide by, checked against brute-force counts on small batches."""
import os
import subprocess
import sys

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def visible_keys_brute(b):
    """Keys a decode query (the last token of its request) sees, counted one by one."""
    n = 0
    for L in b.kv_len:
        q = int(L) - 1
        for j in range(int(L)):
            if b.window > 0 and not (q - j < b.window or j < b.sink):
                continue
            n += 1
    return n


def test_decode_bytes_count_each_visible_key_once():
    for b in (W.tiny_decode_f32(),
              W.paged_batch(name="bytes-window", seed=3, kv_len=[40, 300, 7], qo_len=1, num_qo_heads=8,
                            num_kv_heads=2, head_dim=64, page_size=16, dtype=W.BF16, causal=True, window=50, sink=4)):
        el = 2 if b.dtype == "bf16" else 4
        keys = visible_keys_brute(b)
        T, Hq, Hk, d = int(b.qo_indptr[-1]), b.num_qo_heads, b.num_kv_heads, b.head_dim
        kv_len = np.asarray(b.kv_len, dtype=np.int64)
        vis = np.minimum(kv_len, b.window + b.sink) if b.window > 0 else kv_len
        pages = int(((vis + b.page_size - 1) // b.page_size).sum())
        want = keys * Hk * 2 * d * el + T * Hq * d * el + T * Hq * (d * 4 + 4) + 4 * pages
        assert bench.decode_bytes(b) == want


def test_prefill_flops_count_unmasked_pairs():
    b = W.paged_batch(name="flops", seed=4, kv_len=[10, 37, 5], qo_len=[4, 37, 1], num_qo_heads=4, num_kv_heads=2,
                      head_dim=64, page_size=16, dtype=W.BF16, causal=True)
    pairs = 0
    for Q, L in zip(np.diff(b.qo_indptr), b.kv_len):
        for i in range(int(Q)):
            qpos = int(L) - int(Q) + i
            pairs += sum(1 for j in range(int(L)) if j <= qpos)
    flops, got_pairs = bench.prefill_flops(b)
    assert got_pairs == pairs
    assert flops == 4 * b.head_dim * b.num_qo_heads * pairs
