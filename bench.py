#!/usr/bin/env python3
"""Benchmark of the paged / block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline: paged GQA decode of a Llama-3-8B-shaped layer (batch 64, 32 q / 8
kv heads, head_dim 128, bf16, page 16, kv lengths lognormal in [512, 8192]).
One step = host plan + plan upload + decode kernel + state merge, i.e. the
whole hot path for one batch; two workspaces alternate so the host plan of
step i+1 and its upload (on a copy stream) overlap the GPU work of step i
(--graph 1 replays each step's run + merge from a graph captured at set-up
instead of launching them).  The KV cache is rotated over four
device copies so no step reads what the previous one left in the 256 MB
Infinity Cache.  ``value`` is algorithmic bytes (visible K/V + q + out +
lse + page ids) per wall-clock step, in TB/s; the timed loop holds the
steps only (no timing events, the garbage collector paused).

Also reported (same JSON line): the decode kernel's roofline (HIP events on
its own stream, in a separate pass after the timed loop), the fp64 oracle
timed on a bounded sample of the same
batch on the host cores, and secondary measurements of the ragged causal
prefill (TFLOP/s vs bf16 MFMA peak), the shared-prefix composable format,
the fused-RoPE streaming decode and a mixed decode + prefill batch in one
launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_item.h", "device.h", "args.h", "layout.h"):
        with open(os.path.join(ROOT, "block_sparse_kv_plan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def decode_bytes(batch, out_bytes=4):
    """Algorithmic HBM bytes of one decode pass: each visible key's K and V rows of every kv
    head, q, out, lse and the page ids read."""
    import numpy as np
    kv = batch.kv_len.astype(np.int64)
    if batch.window > 0:
        vis = np.minimum(kv, batch.window + batch.sink)
    else:
        vis = kv
    el = 2 if batch.dtype == "bf16" else 4
    T = int(batch.qo_indptr[-1])
    kvb = int(vis.sum()) * batch.num_kv_heads * batch.head_dim * 2 * el
    qb = T * batch.num_qo_heads * batch.head_dim * el
    ob = T * batch.num_qo_heads * (batch.head_dim * out_bytes + 4)
    pages = int(((vis + batch.page_size - 1) // batch.page_size).sum()) * 4
    return kvb + qb + ob + pages


def prefill_flops(batch):
    """4 d Hq flops per unmasked (query, key) pair of a causal, bottom-right aligned prefill."""
    import numpy as np
    Q = batch.qo_len.astype(np.int64)
    P = batch.kv_len.astype(np.int64) - Q
    pairs = int((Q * P + Q * (Q + 1) // 2).sum())
    return 4 * batch.head_dim * batch.num_qo_heads * pairs, pairs


def make_attention(batch, tile_q, out_dtype, device, **kw):
    import block_sparse_kv_plan_amd as bsk
    from block_sparse_kv_plan_amd.attention import BatchAttention
    rope_mode = {"none": bsk.ROPE_NONE, "streaming": bsk.ROPE_STREAMING, "absolute": bsk.ROPE_ABSOLUTE}[batch.rope]
    args = dict(
        device=device, num_qo_heads=batch.num_qo_heads, num_kv_heads=batch.num_kv_heads, head_dim=batch.head_dim,
        dtype=bsk.DTYPE_BF16 if batch.dtype == "bf16" else bsk.DTYPE_F32, out_dtype=out_dtype,
        kv_mode=bsk.KV_DENSE if batch.kv_mode == "dense" else bsk.KV_PAGED,
        page_size=batch.page_size if batch.kv_mode == "paged" else 16, causal=batch.causal, window=batch.window,
        sink=batch.sink, rope_mode=rope_mode, rope_theta=batch.rope_theta, sm_scale=batch.sm_scale,
        tile_q=tile_q, max_batch=max(1, batch.batch_size))
    args.update(kw)
    return BatchAttention.create(**args)


class Runner:
    """Device copies of one batch plus two alternating plan workspaces.  upload="stream" (default)
    uploads each step's plan on the kernels' own stream; upload="copy" puts it on a copy stream that
    the kernels wait for (on the Llama-3 decode ~0.7 us per step slower: a cross-stream wait, which
    also costs ~13 us of host time); upload="merge" defers each plan's upload into the launch of
    the previous step's merge (bsk_merge_states_upload), so a step is plan, run, and the merge of
    the previous step carrying this step's upload; flush() then merges the last run."""

    def __init__(self, batch, tile_q, copies, device, out_dtype=0, graphs=False, upload="stream", **plan_kw):
        import torch

        import block_sparse_kv_plan_amd as bsk
        from block_sparse_kv_plan_amd.attention import tensors_for
        from workloads.device import rope_positions_needed
        from workloads.device import upload as upload_batch
        if upload not in ("copy", "stream", "merge"):
            raise ValueError(f"upload must be 'copy', 'stream' or 'merge', not {upload!r}")
        if upload == "merge" and graphs:
            raise ValueError("graph replay holds the run and its merge; upload='merge' merges separately")
        self._pending = None  # (workspace, tensors) of a run whose merge is still to come
        self.batch = batch
        self.upload = upload
        self.attn = [make_attention(batch, tile_q, out_dtype, device, **plan_kw) for _ in range(2)]
        T = int(batch.qo_indptr[-1])
        o_dt = torch.bfloat16 if out_dtype == bsk.DTYPE_BF16 else torch.float32
        # one output pair per KV copy, so that consecutive steps never write the same buffers
        self.outs = [(torch.zeros((T, batch.num_qo_heads, batch.head_dim), dtype=o_dt, device=device),
                      torch.zeros((T, batch.num_qo_heads), dtype=torch.float32, device=device))
                     for _ in range(copies)]
        self.out, self.lse = self.outs[0]
        self.rope = None
        if batch.rope != "none":
            n_pos = rope_positions_needed(batch)
            self.rope = torch.empty((n_pos, batch.head_dim // 2, 2), dtype=torch.float32, device=device)
            bsk.rope_table(self.rope, n_pos, batch.head_dim, batch.rope_theta, torch.cuda.current_stream())
        self.dev = []
        first = upload_batch(batch, device=device)
        self.kv_indptr = first["kv_indptr"]
        self.dev.append(first)
        for _ in range(copies - 1):
            self.dev.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in first.items()})
        self.tensors = [tensors_for(self.attn[0].problem, d["q"], d["k"], d["v"], o, l,
                                    page_indices=d["pages"], rope=self.rope) for d, (o, l) in zip(self.dev, self.outs)]
        # run + merge of every (workspace, KV copy) pair a step uses, captured once (each workspace
        # needs a plan before its launches can be recorded; later plans reuse the captures)
        self.graphs = None
        if graphs:
            stream = torch.cuda.current_stream()
            for a in self.attn:
                a.plan(batch.qo_indptr, batch.kv_len, self.kv_indptr, stream=stream)
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            self.graphs = {(w, c): self.attn[w].capture(self.tensors[c], side)
                           for w in range(2) for c in range(copies) if (w - c) % math.gcd(2, copies) == 0}
            torch.cuda.synchronize()

    def step(self, i, stream, copy_stream=None):
        """One pass of the hot path: host plan + upload (on the copy stream when given), the
        attention kernel, then the split-KV state merge (replayed from a graph when captured)."""
        a = self.attn[i % 2]
        c = i % len(self.tensors)
        if self.upload == "merge":
            a.plan(self.batch.qo_indptr, self.batch.kv_len, self.kv_indptr, stream=stream, defer_upload=True)
            if self._pending is not None:
                self._pending[0].merge(self._pending[1], stream, upload_next=a)
            else:
                a.upload(stream)
            a.run(self.tensors[c], stream=stream, merge=False)
            self._pending = (a, self.tensors[c])
            return
        a.plan(self.batch.qo_indptr, self.batch.kv_len, self.kv_indptr, stream=stream, copy_stream=copy_stream)
        if self.graphs is not None:
            a.replay(self.graphs[(i % 2, c)], stream)
        else:
            a.run(self.tensors[c], stream=stream)

    def flush(self, stream):
        """The merge still owed by the last step (upload="merge"); nothing otherwise."""
        if self._pending is not None:
            self._pending[0].merge(self._pending[1], stream)
            self._pending = None


WARM_S = 0.25  # sustained load before a secondary leg's timing (MFMA-bound kernels run ~20% slower for
               # the first ~50 ms of back-to-back launches while the clock ramps; HBM-bound ones do not)


def keep_busy(launch, seconds):
    """Call launch(i) back to back until `seconds` of wall time have passed, synchronising every
    eight calls so that the time counted is time the GPU spent busy."""
    import torch
    t_end = time.perf_counter() + seconds
    i = 0
    while True:
        for _ in range(8):
            launch(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return


def wall_clock(runner, steps, warmup, warm_s=0.0):
    """Wall time per step over `steps` back-to-back steps after `warmup` untimed ones.

    Plans are uploaded as the runner says (on a copy stream or on the kernels' stream).  Nothing
    but the steps runs in the timed loop: no timing events (kernel durations come from a separate
    pass, kernel_durations()), and the Python garbage collector is paused, so the loop's contents
    do not depend on `steps`.  Host stamps after each step's submission show whether the host kept
    ahead of the GPU.  warm_s > 0 adds that much sustained load after the warm-up steps."""
    import gc

    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream() if runner.upload == "copy" else None
    stamps = np.zeros(steps)
    gc.collect()  # before the warm-up: a collection takes milliseconds, which the GPU would spend idle
    gc.disable()
    try:
        done = [0]

        def one(_):
            runner.step(done[0], stream, copy_stream=copy_stream)
            done[0] += 1

        for i in range(warmup):
            one(i)
        if warm_s > 0:
            keep_busy(one, warm_s)
        runner.flush(stream)
        torch.cuda.synchronize()
        first = done[0]
        t0 = time.perf_counter()
        for i in range(steps):
            runner.step(first + i, stream, copy_stream=copy_stream)
            stamps[i] = time.perf_counter()
        runner.flush(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    finally:
        gc.enable()
    host = np.diff(np.concatenate([[t0], stamps])) * 1e6
    return {"wall_s": (t1 - t0) / steps, "host_submit_us_median": round(float(np.median(host)), 1),
            "host_submit_us_max": round(float(host.max()), 1), "drain_us": round((t1 - stamps[-1]) * 1e6, 1)}


def kernel_durations(runner, reps, warm_s=0.0):
    """The attention kernel's launch duration from HIP events recorded on its own stream right
    around it, over `reps` launches on the last plans (KV copies rotating as in the timed loop).
    Runs after the wall-clock loop, so its events never share a queue with it.  warm_s > 0 first
    keeps the GPU busy with the same launches for that long."""
    import torch
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if warm_s > 0:
        keep_busy(lambda i: runner.attn[i % 2].run(runner.tensors[i % len(runner.tensors)], stream=stream), warm_s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(3):
        runner.attn[i % 2].run(runner.tensors[i % len(runner.tensors)], stream=stream)
    for i, (e0, e1) in enumerate(evs):
        a = runner.attn[i % 2]
        t = runner.tensors[i % len(runner.tensors)]
        e0.record(stream)
        a.run(t, stream=stream, merge=False, wait_upload=False)
        e1.record(stream)
        a.merge(t, stream)
    torch.cuda.synchronize()
    k = sorted(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)
    pct = lambda q: k[min(len(k) - 1, int(q * len(k)))]
    return {"kernel_s_mean": sum(k) / len(k), "kernel_s_median": pct(0.5), "kernel_s_p10": pct(0.1),
            "kernel_s_p90": pct(0.9), "kernel_s_min": k[0], "samples": len(k)}


def plan_host_us(runner, calls=50):
    """Mean host time of the C++ plan for the runner's batch (no upload)."""
    import numpy as np

    import block_sparse_kv_plan_amd as bsk
    b, a = runner.batch, runner.attn[0]
    qo = np.ascontiguousarray(b.qo_indptr, dtype=np.int32)
    kl = np.ascontiguousarray(b.kv_len, dtype=np.int32)
    ki = np.ascontiguousarray(runner.kv_indptr, dtype=np.int32)
    host = np.zeros(a.host_ws.numel(), dtype=np.uint8)  # a private buffer: no upload is in flight from it
    bsk.plan(a.problem, qo, kl, ki, host)
    t0 = time.perf_counter()
    for _ in range(calls):
        bsk.plan(a.problem, qo, kl, ki, host)
    return round((time.perf_counter() - t0) / calls * 1e6, 1)


def cpu_baseline(batch, budget_s=15.0):
    """fp64 oracle on the host: requests one at a time until the budget is used; the rate is
    scaled to the metric's unit (algorithmic bytes / oracle seconds)."""
    import copy

    import numpy as np

    from threadpoolctl import threadpool_limits

    import oracle
    from oracle.attention import PagedKV
    kp, vp, idx = batch.host_pools()  # host view of the cache, built once outside the timed calls
    kv = PagedKV(kp, vp, batch.kv_page_indptr, idx, batch.page_size)
    done, t_used, bytes_done = 0, 0.0, 0
    limits = threadpool_limits(limits=1)  # the oracle's one BLAS product runs single-threaded too
    for r in range(batch.batch_size):
        sub = copy.copy(batch)
        t0 = time.perf_counter()
        oracle.attention(batch.q, batch.qo_indptr, batch.kv_len, kv, batch.num_kv_heads, batch.sm_scale,
                         causal=batch.causal, window=batch.window, sink=batch.sink, rope=batch.rope,
                         rope_theta=batch.rope_theta,
                         tokens=list(range(int(batch.qo_indptr[r]), int(batch.qo_indptr[r + 1]))))
        t_used += time.perf_counter() - t0
        sub.kv_len = batch.kv_len[r:r + 1]
        sub.qo_indptr = np.array([0, int(batch.qo_indptr[r + 1] - batch.qo_indptr[r])])
        bytes_done += decode_bytes(sub)
        done += 1
        if t_used > budget_s:
            break
    limits.restore_original_limits()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass
    return {"value": bytes_done / t_used / 1e12, "unit": "TB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {batch.batch_size} requests of the same batch (fp64 numpy, BLAS held to "
                      f"one thread for its two matrix products), {t_used:.1f} s",
            "cpu": model, "cores_available": len(os.sched_getaffinity(0)), "blas_threads": 1}


def load_traffic(name, launches_bytes):
    """Measured HBM bytes of the decode kernel from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def ceilings(device):
    """What the vendor stack reaches on this GPU for the two bounds: a large bf16 GEMM through
    torch.matmul (hipBLASLt) and a device-to-device copy (bytes read + written).  Context for the
    roofline fractions, which are quoted against the published peaks."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    out = {}
    n = 8192
    a = torch.randn((n, n), device=device).to(torch.bfloat16)
    b = torch.randn((n, n), device=device).to(torch.bfloat16)
    c = torch.empty((n, n), device=device, dtype=torch.bfloat16)
    keep_busy(lambda i: torch.matmul(a, b, out=c), WARM_S)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    out["bf16_gemm_8192_tflops"] = round(2 * n ** 3 / s / 1e12, 1)
    out["bf16_gemm_frac_of_peak"] = round(2 * n ** 3 / s / 1e12 / BF16_PEAK_TFLOPS, 4)
    del a, b, c
    src = torch.empty(1 << 31, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    out["copy_2gib_gbs"] = round(2 * src.numel() / s / 1e9, 1)
    out["copy_frac_of_peak"] = round(2 * src.numel() / s / 1e9 / HBM_PEAK_GBS, 4)
    del dst
    # streaming read: the library's read hook (every 16-byte piece once, non-temporal loads), best of
    # four grid sizes (more workgroups than three per CU oversubscribe the memory system: a sweep read
    # 7.0 TB/s at two or three per CU, 5.8 at four)
    import block_sparse_kv_plan_amd as bsk
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    best = 0.0
    for per_cu in (1, 2, 3, 4):
        grid = cus * per_cu
        sink = torch.empty(grid * 256, dtype=torch.int32, device=device)
        keep_busy(lambda i: bsk.debug_stream_read(src, sink, grid, stream), 0.05)
        e0.record(stream)
        for _ in range(reps):
            bsk.debug_stream_read(src, sink, grid, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3 / reps
        if src.numel() / s / 1e9 > best:
            best, best_grid = src.numel() / s / 1e9, grid
    out["read_2gib_gbs"] = round(best, 1)
    out["read_frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
    out["read_grid"] = best_grid
    # the same read over the Llama-3 decode's algorithmic bytes (one launch of that size, with its
    # fixed start and drain), three disjoint slices of the buffer in turn (each read last two launches
    # earlier, 1.4 GB before: not in the 256 MB Infinity Cache)
    nb = 695809520 // 16 * 16
    sink = torch.empty(best_grid * 256, dtype=torch.int32, device=device)
    views = [src[k * 664 * 2**20:k * 664 * 2**20 + nb] for k in range(3)]  # 664 MiB apart, each nb bytes
    assert all(v.numel() == nb for v in views)
    keep_busy(lambda i: bsk.debug_stream_read(views[i % 3], sink, best_grid, stream), 0.05)
    e0.record(stream)
    for i in range(reps * 3):
        bsk.debug_stream_read(views[i % 3], sink, best_grid, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / (reps * 3)
    out["read_decode_volume_us"] = round(s * 1e6, 1)
    out["read_decode_volume_gbs"] = round(nb / s / 1e9, 1)
    # the paged decode's access pattern: the 2 GiB buffer's 4 KB blocks (one kv head's 16 keys of K or V
    # at d = 128) in a seeded random order, two blocks in flight per wave, best of four grid sizes
    n_blk = src.numel() // 4096
    order = torch.from_numpy(np.random.default_rng(4096).permutation(n_blk).astype(np.int32)).to(device)
    best_b = 0.0
    for per_cu in (1, 2, 3, 4):
        grid = cus * per_cu
        sink = torch.empty(grid * 256, dtype=torch.int32, device=device)
        keep_busy(lambda i: bsk.debug_block_read(src, order, sink, grid, stream), 0.05)
        e0.record(stream)
        for _ in range(reps):
            bsk.debug_block_read(src, order, sink, grid, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3 / reps
        if src.numel() / s / 1e9 > best_b:
            best_b, best_bgrid = src.numel() / s / 1e9, grid
    out["read_random_4k_blocks_gbs"] = round(best_b, 1)
    out["read_random_4k_blocks_frac_of_peak"] = round(best_b / HBM_PEAK_GBS, 4)
    out["read_random_4k_blocks_grid"] = best_bgrid
    out["note"] = ("GEMM: 2 n^3 flop per torch.matmul, n = 8192; copy: 2 GiB read + 2 GiB written per copy; "
                   "read: bsk_debug_stream_read over 2 GiB, best of 1-4 workgroups per CU, and over the Llama-3 "
                   "decode's 695.8 MB per launch; random 4 KB blocks: bsk_debug_block_read over the 2 GiB "
                   "buffer's blocks in a seeded random order (the paged decode's access pattern)")
    del src
    return out


def mixed_leg(device, reps):
    """GPU time of one mixed batch (64 decode requests and 4 prefill chunks): the mixed launch
    (both tile classes in one persistent kernel, then the state merge) against the decode
    kernel over the decode requests followed by the prefill kernel over the prefill requests
    (each with its merge).  Plans are built once; HIP events on the launch stream."""
    import numpy as np
    import torch

    import block_sparse_kv_plan_amd as bsk
    import workloads as W
    from block_sparse_kv_plan_amd.attention import tensors_for
    from workloads.device import upload
    b = W.mixed()
    dec = b.qo_len == 1
    parts = {"mixed": (b, dict(tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE))}
    for name, sel, tq in (("decode", dec, bsk.TILE_DECODE), ("prefill", ~dec, bsk.TILE_PREFILL)):
        sub = W.paged_batch(name=f"mixed_{name}_part", seed=7, kv_len=b.kv_len[sel], qo_len=b.qo_len[sel],
                            num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                            page_size=b.page_size, dtype=b.dtype, causal=True)
        parts[name] = (sub, dict(tile_q=tq))
    stream = torch.cuda.current_stream()
    runs = {}
    for name, (bb, kw) in parts.items():
        tq = kw.pop("tile_q")
        attn = make_attention(bb, tq, 0, device, **kw)
        d = upload(bb, device=device)
        T = int(bb.qo_indptr[-1])
        out = torch.empty((T, bb.num_qo_heads, bb.head_dim), dtype=torch.float32, device=device)
        lse = torch.empty((T, bb.num_qo_heads), dtype=torch.float32, device=device)
        t = tensors_for(attn.problem, d["q"], d["k"], d["v"], out, lse, page_indices=d["pages"])
        attn.plan(bb.qo_indptr, bb.kv_len, d["kv_indptr"], stream=stream)
        runs[name] = (attn, t, d, out, lse)

    def go(names):
        for n in names:
            attn, t = runs[n][0], runs[n][1]
            attn.run(t, stream=stream)

    res = {}
    for label, names in (("one_launch", ["mixed"]), ("two_launches", ["decode", "prefill"])):
        keep_busy(lambda i: go(names), WARM_S)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e in evs:
            e[0].record(stream)
            go(names)
            e[1].record(stream)
        torch.cuda.synchronize()
        res[label] = sum(e[0].elapsed_time(e[1]) for e in evs) / reps * 1e3
    info = runs["mixed"][0].info
    flops, _ = prefill_flops(parts["prefill"][0])
    nbytes = decode_bytes(parts["decode"][0])
    return {
        "workload": "mixed_decode_prefill_bf16: 64 decode requests (kv lognormal [512,8192]) + 4 prefill chunks "
                    "(lognormal [256,2048] new tokens after uniform [0,2048] cached), 32q/8kv, d128, page 16",
        "one_launch_us": round(res["one_launch"], 2), "two_launches_us": round(res["two_launches"], 2),
        "speedup": round(res["two_launches"] / res["one_launch"], 3),
        "mixed_items": info.num_items, "mixed_workers": info.num_workers, "mixed_merges": info.num_merge,
        "decode_part_bytes": nbytes, "prefill_part_flops": flops,
        "note": "kernel + merge GPU time per batch, plans built once; the parts of the two-launch run are "
                "separate batches of the same lengths and shapes"}


def stride_cases(prefill_tile):
    """(name, batch factory, tile_q, plan kwargs) of the K/V stride-specialisation case set: decode batch
    sizes, head dims, GQA groups, dense KV, the fused-RoPE window decode, ragged prefill with both tile
    classes and head dim 64, and the mixed decode + prefill launch."""
    import block_sparse_kv_plan_amd as bsk
    import workloads as W
    D, P = bsk.TILE_DECODE, bsk.TILE_PREFILL
    lens = lambda B, seed=2: W.llama3_decode_lengths(seed=seed, batch=B)[1]
    cases = [(f"decode_b{B}", (lambda B=B: W.llama3_decode(batch=B)), D, {}) for B in (8, 16, 32, 64, 128)]
    cases += [
        ("decode_d64_b64", lambda: W.paged_batch(name="decode_d64", seed=21, kv_len=lens(64, 21), qo_len=1,
                                                  num_qo_heads=32, num_kv_heads=8, head_dim=64, page_size=16,
                                                  dtype=W.BF16, causal=True), D, {}),
        ("decode_gqa8_b32", lambda: W.paged_batch(name="decode_gqa8", seed=22, kv_len=lens(32, 22), qo_len=1,
                                                   num_qo_heads=64, num_kv_heads=8, head_dim=128, page_size=16,
                                                   dtype=W.BF16, causal=True), D, {}),
        ("decode_page64_b32", lambda: W.paged_batch(name="decode_page64", seed=23, kv_len=lens(32, 23), qo_len=1,
                                                     num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
                                                     dtype=W.BF16, causal=True), D, dict(tile_kv=64)),
        ("decode_dense_b32", lambda: W.dense_batch(name="decode_dense", seed=24, kv_len=lens(32, 24), qo_len=1,
                                                    num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype=W.BF16,
                                                    causal=True), D, {}),
        ("rope_window_decode", W.streaming_rope_decode, D, dict(split_factor=2)),
        ("prefill_ragged_t256", W.ragged_prefill, 256, {}),
        ("prefill_ragged_t128", W.ragged_prefill, P, {}),
        ("prefill_d64", lambda: W.paged_batch(name="prefill_d64", seed=25, kv_len=W.ragged_prefill_lengths(seed=25)[1],
                                              qo_len=W.ragged_prefill_lengths(seed=25)[0], num_qo_heads=32,
                                              num_kv_heads=8, head_dim=64, page_size=16, dtype=W.BF16, causal=True),
         prefill_tile, {}),
        ("mixed_batch", W.mixed, P, dict(decode_tile_q=D)),
    ]
    return cases


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="profiling aid: run just this workload (decode|prefill|append|strides|composable|rope|mixed|ceilings)")
    ap.add_argument("--prefill-tile", type=int, default=None, choices=(128, 256),
                    help="query-row tile of the prefill kernel for both the ragged prefill and the composable "
                         "prefix (default: 256 for the ragged prefill, 128 for the prefix)")
    ap.add_argument("--decode-split", type=int, default=None, help="plan split_factor of the decode workload")
    ap.add_argument("--decode-min-chunk", type=int, default=None, help="plan min_chunk (keys) of the decode workload")
    ap.add_argument("--decode-overhead", type=int, default=None, help="plan item_overhead (keys) of the decode workload")
    ap.add_argument("--fused-merge", type=int, choices=(0, 1), default=None,
                    help="merge split units in-kernel (1) or with the separate merge kernel (0) on the decode-class "
                         "workloads (Llama-3 decode, streaming RoPE decode)")
    ap.add_argument("--graph", type=int, choices=(0, 1), default=0,
                    help="replay each step's run + merge from a graph captured at set-up (1) or launch them "
                         "directly (0, default: two direct launches measured faster than one graph launch)")
    ap.add_argument("--upload", choices=("copy", "stream", "merge"), default="merge",
                    help="where the Llama-3 decode leg uploads each plan: in the previous step's merge launch "
                         "(default), on the kernels' own stream, or on a copy stream the kernels wait for")
    ap.add_argument("--rope-upload", choices=("stream", "merge"), default="merge",
                    help="where the streaming-RoPE leg uploads each plan: in the previous step's merge launch "
                         "(default) or on the kernels' own stream")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="profiling aid: first run one plain device copy of this many MiB, the reference that "
                         "scales hardware byte counters")
    args = ap.parse_args()
    # query-row tile of the ragged-prefill legs (256-row items: eight waves share each K/V tile)
    # and of the composable's dense prefix (128-row items: twice the workers for 64 branch tokens)
    prefill_tile = args.prefill_tile or 256
    prefix_tile = args.prefill_tile or 128
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this build has no multi-GPU "
              "path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_kv_plan_amd as bsk
    import workloads as W

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst
    result = {}
    secondary = {}

    if args.only in ("", "decode"):
        log("decode: generating the Llama-3-8B-shaped batch")
        b = W.llama3_decode()
        nbytes = decode_bytes(b)
        dkw = {k: v for k, v in (("split_factor", args.decode_split), ("min_chunk", args.decode_min_chunk),
                                  ("item_overhead", args.decode_overhead), ("fused_merge", args.fused_merge))
               if v is not None}
        # a replayed graph holds the run and its merge, so it uploads in-stream instead of in the merge
        up_mode = "stream" if args.graph and args.upload == "merge" else args.upload
        runner = Runner(b, bsk.TILE_DECODE, copies=4, device=device, graphs=bool(args.graph), upload=up_mode, **dkw)
        log(f"decode: {int(b.kv_len.sum())} keys, {nbytes / 1e9:.3f} GB per step; timing {args.steps} steps")
        m = wall_clock(runner, args.steps, args.warmup)
        m.update(kernel_durations(runner, max(20, min(args.steps, 100))))
        info = runner.attn[0].info
        achieved = nbytes / m["kernel_s_mean"] / 1e9
        plan_us = plan_host_us(runner)
        traffic = load_traffic("decode_llama3", nbytes)
        step_desc = {"copy": "plan + upload on a copy stream + run + merge",
                     "stream": "plan + upload on the kernels' stream + run + merge",
                     "merge": "plan + run + merge, each plan's upload made in the launch of the previous step's "
                              "merge; the first upload and the last merge on their own"}[up_mode]
        result = {
            "metric": "paged decode HBM TB/s (% of 8 TB/s peak); ragged prefill TFLOPS (% MFMA peak)",
            "value": round(nbytes / m["wall_s"] / 1e12, 4),
            "unit": "TB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(m["wall_s"] * 1e3, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "llama3_8b_paged_decode_bf16", "batch": 64, "num_qo_heads": 32,
                       "num_kv_heads": 8, "head_dim": 128, "page_size": 16,
                       "kv_len": "lognormal clipped to [512, 8192]", "total_kv_tokens": int(b.kv_len.sum()),
                       "out_dtype": "f32", "num_workers": info.num_workers, "items": info.num_items,
                       "chunk": info.chunk, "merges": info.num_merge,
                       "plan_imbalance": round(info.max_load / max(1.0, info.total_cost / info.num_workers), 3),
                       "plan_host_us": plan_us, "graph_replay": bool(args.graph),
                       "parallelism": "single GPU"},
            "timing": {"protocol": f"wall clock over the timed steps ({step_desc}; "
                                   "no events in the loop, garbage collector paused); kernel durations from HIP "
                                   "events around the kernel in a separate pass afterwards",
                       "host_submit_us_median": m["host_submit_us_median"],
                       "host_submit_us_max": m["host_submit_us_max"], "drain_us": m["drain_us"]},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic, "kernel": "decode_kernel<bf16,128,paged>",
                         "kernel_us_mean": round(m["kernel_s_mean"] * 1e6, 2),
                         "kernel_us_median": round(m["kernel_s_median"] * 1e6, 2),
                         "kernel_us_p10": round(m["kernel_s_p10"] * 1e6, 2),
                         "kernel_us_p90": round(m["kernel_s_p90"] * 1e6, 2),
                         "event_samples": m["samples"],
                         "algorithmic_bytes_per_launch": nbytes},
        }
        if not args.no_cpu:
            log("decode: timing the fp64 oracle on a bounded sample")
            result["cpu_baseline"] = cpu_baseline(b)
        del runner
        torch.cuda.empty_cache()

    if not args.no_secondary and args.only in ("", "prefill"):
        log("prefill: ragged causal prefill with append")
        b = W.ragged_prefill()
        flops, pairs = prefill_flops(b)
        runner = Runner(b, prefill_tile, copies=1, device=device)
        m = wall_clock(runner, max(5, args.steps // 10), 3, warm_s=WARM_S)
        m.update(kernel_durations(runner, max(10, min(args.steps // 5, 40)), warm_s=WARM_S))
        tf = flops / m["kernel_s_mean"] / 1e12
        secondary["ragged_prefill"] = {
            "workload": "ragged_causal_prefill_append_bf16: 16 requests, q lognormal [128,4096] after "
                        "uniform [0,2048] cached keys, 32q/8kv, d128",
            "tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "kernel_us_mean": round(m["kernel_s_mean"] * 1e6, 1), "step_ms": round(m["wall_s"] * 1e3, 3),
            "unmasked_pairs": pairs, "flops": flops, "tile_q": prefill_tile,
            "num_workers": runner.attn[0].info.num_workers, "items": runner.attn[0].info.num_items}
        del runner
        torch.cuda.empty_cache()

    if not args.no_secondary and args.only in ("", "append"):
        log("append: new tokens' K/V of the ragged prefill into the paged cache; chunked prefill")
        from block_sparse_kv_plan_amd.attention import BatchAttention, chunked_prefill, pool_strides
        from workloads.device import upload
        b = W.ragged_prefill()
        du = upload(b, device=device)
        new = b.qo_len.astype(np.int64)
        prefix = b.kv_len.astype(np.int64) - new
        T = int(new.sum())
        el = 2
        kn = torch.randn((T, b.num_kv_heads, b.head_dim), device=device).to(torch.bfloat16)
        vn = torch.randn((T, b.num_kv_heads, b.head_dim), device=device).to(torch.bfloat16)
        prob = make_attention(b, bsk.TILE_PREFILL, 0, device).problem
        app = torch.as_tensor(np.concatenate([[0], np.cumsum(new)]).astype(np.int32), device=device)
        kvl = torch.as_tensor(b.kv_len.astype(np.int32), device=device)
        pip = torch.as_tensor(du["kv_indptr"], device=device)
        stream = torch.cuda.current_stream()

        def do_append():
            bsk.append_paged_kv(prob, b.batch_size, T, app, kvl, pip, du["pages"], kn, vn, kn.stride(0),
                                kn.stride(1), du["k"], du["v"], pool_strides(du["k"]), pool_strides(du["v"]), stream)
        for _ in range(3):
            do_append()
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            do_append()
        e1.record(stream)
        torch.cuda.synchronize()
        app_s = e0.elapsed_time(e1) * 1e-3 / reps
        app_bytes = 2 * 2 * T * b.num_kv_heads * b.head_dim * el  # K and V, read and written
        secondary["append_paged_kv"] = {
            "workload": f"the ragged prefill's {T} new tokens, 8 kv heads, d128, bf16, page 16",
            "us": round(app_s * 1e6, 2), "gbs": round(app_bytes / app_s / 1e9, 1),
            "frac_of_hbm_peak": round(app_bytes / app_s / 1e9 / HBM_PEAK_GBS, 4), "bytes": app_bytes}
        flops, _ = prefill_flops(b)
        attn = BatchAttention.create(device=device, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                                     head_dim=b.head_dim, dtype=bsk.DTYPE_BF16, page_size=b.page_size, causal=True,
                                     tile_q=prefill_tile, max_batch=b.batch_size)
        out = torch.empty((T, b.num_qo_heads, b.head_dim), dtype=torch.float32, device=device)
        lse = torch.empty((T, b.num_qo_heads), dtype=torch.float32, device=device)
        chunk = 4096
        chunked_prefill(attn, du["q"], kn, vn, out, lse, du["k"], du["v"], du["pages"], du["kv_indptr"], prefix,
                        new, chunk)
        torch.cuda.synchronize()
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            chunked_prefill(attn, du["q"], kn, vn, out, lse, du["k"], du["v"], du["pages"], du["kv_indptr"], prefix,
                            new, chunk)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / reps
        secondary["chunked_prefill"] = {
            "workload": f"the ragged prefill run as steps of {chunk} new tokens (append + plan + prefill + merge "
                        f"per step), tile_q {prefill_tile}",
            "steps": (T + chunk - 1) // chunk, "wall_ms": round(wall * 1e3, 3),
            "tflops_incl_host_steps": round(flops / wall / 1e12, 1)}
        del attn, du
        torch.cuda.empty_cache()

    if not args.no_secondary and args.only in ("", "strides"):
        log("strides: equal-stride (shared address) kernels vs independent K/V stride kernels, same data")
        ab = {}
        for name, make, tq, kw in stride_cases(prefill_tile):
            b = make()
            runners = [Runner(b, tq, copies=2, device=device, independent_kv_strides=ind, **kw) for ind in (0, 1)]
            for runner in runners:
                for a in runner.attn:
                    a.plan(b.qo_indptr, b.kv_len, runner.kv_indptr, stream=torch.cuda.current_stream())
            # the two variants alternate in three rounds after sustained load, so neither sees a colder GPU
            reps = 10 if tq == bsk.TILE_DECODE else 4
            tot = [0.0, 0.0]
            for rnd in range(3):
                for v, runner in enumerate(runners):
                    tot[v] += kernel_durations(runner, reps, warm_s=WARM_S if rnd == 0 and v == 0 else 0.0)[
                        "kernel_s_mean"]
            us = [t / 3 * 1e6 for t in tot]
            del runners
            torch.cuda.empty_cache()
            ab[name] = {"equal_strides_us": round(us[0], 2), "independent_strides_us": round(us[1], 2),
                        "speedup": round(us[1] / us[0], 4)}
            log(f"  strides {name}: {us[1] / us[0]:.4f}x")
        sp = [v["speedup"] for v in ab.values()]
        secondary["kv_stride_specialization"] = {
            "cases": ab, "geomean_speedup": round(math.exp(sum(math.log(x) for x in sp) / len(sp)), 4),
            "n_cases": len(sp), "pages_geomean_b200": 1.0456,
            "note": "kernel time with K and V sharing page/head/token strides (one address per key, V at the K-to-V "
                    "distance) against the general kernels forced by independent_kv_strides=1 on the same data; "
                    "the pages report a 1.0456x geomean over 30 cases on B200"}

    if not args.no_secondary and args.only in ("", "rope"):
        log("rope: long-context streaming decode with fused RoPE, window 4096 + 4 sinks")
        b = W.streaming_rope_decode()
        nbytes = decode_bytes(b)
        # Each unit sees 4100 keys (the window and the sinks).  Split factor 2 lets the 512-key chunk
        # minimum bind: 512 keys are 32 blocks, eight for each of a worker's four waves, where the
        # default's 528-key chunks give one wave a ninth block.  The unfused baseline uses the same plan.
        rplan = {"split_factor": 2}
        rkw = dict(rplan) if args.fused_merge is None else dict(rplan, fused_merge=args.fused_merge)
        # a host-bound step (~38 us of GPU work): the plan goes up on the kernels' own stream, in its own
        # launch or in the previous step's merge launch (a replayed graph holds the merge: in-stream)
        r_up = "stream" if args.graph else args.rope_upload
        runner = Runner(b, bsk.TILE_DECODE, copies=3, device=device, graphs=bool(args.graph), upload=r_up, **rkw)
        m = wall_clock(runner, args.steps, args.warmup, warm_s=WARM_S)
        m.update(kernel_durations(runner, max(20, min(args.steps, 100)), warm_s=WARM_S))
        secondary["streaming_rope_decode"] = {
            "workload": "streaming_rope_window_sink_decode_bf16: batch 8, kv uniform [32768,131072], 64q/8kv, "
                        "d128, window 4096 + 4 sinks, RoPE theta 5e5 in-kernel",
            "kernel_gbs": round(nbytes / m["kernel_s_mean"] / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / m["kernel_s_mean"] / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_us_mean": round(m["kernel_s_mean"] * 1e6, 2), "step_us": round(m["wall_s"] * 1e6, 1),
            "host_submit_us_median": m["host_submit_us_median"], "plan_upload": {"stream": "kernels' stream", "merge": "previous step's merge launch"}[r_up],
            "algorithmic_bytes": nbytes}
        # unfused reference point: rotate the visible keys and the query into scratch, then a plain
        # windowed decode over (rotated K, V); same bytes credited as the fused kernel's
        from block_sparse_kv_plan_amd.attention import tensors_for
        d0 = runner.dev[0]
        k_out = torch.empty_like(d0["k"])
        q_out = torch.empty_like(d0["q"])
        i32 = lambda x: torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)
        qo_d, kvl_d, pip_d = i32(b.qo_indptr), i32(b.kv_len), i32(runner.kv_indptr)
        rprob = runner.attn[0].problem
        t_rot = tensors_for(rprob, d0["q"], d0["k"], d0["v"], runner.out, runner.lse, page_indices=d0["pages"],
                            rope=runner.rope)
        plain = make_attention(b, bsk.TILE_DECODE, 0, device, rope_mode=bsk.ROPE_NONE, **rplan)
        t_plain = tensors_for(plain.problem, q_out, k_out, d0["v"], runner.out, runner.lse, page_indices=d0["pages"])
        stream = torch.cuda.current_stream()
        plain.plan(b.qo_indptr, b.kv_len, runner.kv_indptr, stream=stream)
        reps = max(10, args.steps // 2)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 3)]
        for i in range(reps + 3):
            evs[i][0].record(stream)
            bsk.rope_apply(rprob, b.batch_size, int(b.kv_len.max()), qo_d, kvl_d, pip_d, t_rot, q_out,
                           q_out.stride(0), q_out.stride(1), k_out, stream)
            evs[i][1].record(stream)
            plain.run(t_plain, stream=stream, merge=False)
            evs[i][2].record(stream)
        torch.cuda.synchronize()
        rot_us = sum(e[0].elapsed_time(e[1]) for e in evs[3:]) / reps * 1e3
        dec_us = sum(e[1].elapsed_time(e[2]) for e in evs[3:]) / reps * 1e3
        fused_us = m["kernel_s_mean"] * 1e6
        secondary["unfused_rope_baseline"] = {
            "workload": "the streaming-RoPE decode above, RoPE applied by a separate pass (visible keys and the "
                        "query rotated into scratch, bf16), then the plain windowed decode",
            "rotate_us": round(rot_us, 2), "decode_us": round(dec_us, 2), "unfused_us": round(rot_us + dec_us, 2),
            "fused_us": round(fused_us, 2), "fused_speedup": round((rot_us + dec_us) / fused_us, 3),
            "fused_gbs": round(nbytes / fused_us / 1e3, 1), "unfused_gbs": round(nbytes / (rot_us + dec_us) / 1e3, 1),
            "note": "effective bandwidth = the fused kernel's algorithmic bytes / time (the pages report 1.6-3.7x "
                    "for fused RoPE + attention)"}
        del runner, plain, k_out, q_out
        torch.cuda.empty_cache()

    if not args.no_secondary and args.only in ("", "composable"):
        log("composable: shared 16384-token dense prefix + 64 paged suffixes")
        c = W.shared_prefix()
        from block_sparse_kv_plan_amd.attention import run_composable
        stream = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        n = max(10, args.steps // 2)
        cus = torch.cuda.get_device_properties(device).multi_processor_count
        pb = 16384 * 8 * 128 * 2 * 2
        sb = decode_bytes(c.suffix)
        leg = {"workload": "shared_prefix_composable_bf16: 16384-token dense prefix + 64 paged suffixes uniform "
                           "[128,1024], 32q/8kv, d128",
               "algorithmic_bytes": pb + sb}
        copies = 3  # 3 x 218 MB of K/V rotate, so no repetition finds the last one's in the 256 MB Infinity Cache

        def gpu_us(step):
            keep_busy(step, WARM_S)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                step(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / n

        # sequential: each part on the whole GPU, one after the other; concurrent: each part planned
        # for half the GPU, the suffix on a side stream beside the prefix
        for label, workers, side_stream in (("sequential", (None, None), None), ("concurrent", (cus, cus), side)):
            kw_p = {"num_workers": workers[0]} if workers[0] else {}
            kw_s = {"num_workers": workers[1]} if workers[1] else {}
            pre = Runner(c.prefix, prefix_tile, copies=copies, device=device, **kw_p)
            suf = Runner(c.suffix, bsk.TILE_DECODE, copies=copies, device=device, **kw_s)
            fin_o = torch.empty_like(suf.out)
            fin_l = torch.empty_like(suf.lse)

            a, b = pre.attn[0], suf.attn[0]
            t0 = time.perf_counter()
            a.plan(c.prefix.qo_indptr, c.prefix.kv_len, pre.kv_indptr, stream=stream)
            b.plan(c.suffix.qo_indptr, c.suffix.kv_len, suf.kv_indptr, stream=stream)
            plan_us = (time.perf_counter() - t0) * 1e6

            def one(i):
                k = i % copies
                run_composable(a, pre.tensors[k], pre.outs[k], b, suf.tensors[k], suf.outs[k], fin_o, fin_l,
                               stream=stream, side_stream=side_stream)

            gpu = gpu_us(one)
            leg[label] = {"gpu_us_per_step": round(gpu * 1e6, 1), "effective_gbs": round((pb + sb) / gpu / 1e9, 1),
                          "host_plans_us": round(plan_us, 1), "prefix_workers": a.info.num_workers,
                          "suffix_workers": b.info.num_workers, "launches": 5}
            del pre, suf
            torch.cuda.empty_cache()
        # one launch: the prefix's 128-row items and the suffixes' decode items planned together and run
        # on one persistent grid, then one merge pass (shared_prefix_len). Two target chunks per worker
        # make L_c 1024, which splits the 16384-key prefix into 16 equal chunks; one gives L_c 1152 and a
        # 256-key tail chunk per prefix tile (measured 57-58 against 60 us per launch)
        from block_sparse_kv_plan_amd.attention import BatchAttention, tensors_for
        from workloads.device import upload
        one_attn = BatchAttention.create(device=device, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                                         dtype=bsk.DTYPE_BF16, page_size=16, causal=True, max_batch=64,
                                         tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE,
                                         shared_prefix_len=16384, split_factor=2)
        du = [upload(c.suffix, device=device) for _ in range(copies)]
        pkv = [(torch.from_numpy(c.prefix.dense_k).to(torch.bfloat16).to(device),
                torch.from_numpy(c.prefix.dense_v).to(torch.bfloat16).to(device)) for _ in range(copies)]
        one_out = [(torch.empty((64, 32, 128), dtype=torch.float32, device=device),
                    torch.empty((64, 32), dtype=torch.float32, device=device)) for _ in range(copies)]
        one_t = [tensors_for(one_attn.problem, d["q"], d["k"], d["v"], o, l, page_indices=d["pages"], prefix_k=pk,
                             prefix_v=pv) for d, (pk, pv), (o, l) in zip(du, pkv, one_out)]
        t0 = time.perf_counter()
        info = one_attn.plan(c.suffix.qo_indptr, c.suffix.kv_len, du[0]["kv_indptr"], stream=stream)
        plan_us = (time.perf_counter() - t0) * 1e6
        gpu = gpu_us(lambda i: one_attn.run(one_t[i % copies], stream=stream))
        leg["one_launch"] = {"gpu_us_per_step": round(gpu * 1e6, 1), "effective_gbs": round((pb + sb) / gpu / 1e9, 1),
                             "host_plans_us": round(plan_us, 1), "workers": info.num_workers, "items": info.num_items,
                             "merges": info.num_merge, "chunk": info.chunk, "launches": 2}
        del one_attn, du, pkv, one_out
        torch.cuda.empty_cache()
        leg["note"] = ("GPU time per step, plans built once (they depend only on lengths), three copies of the "
                       "K/V rotating; sequential / concurrent: prefix run + suffix run (each with its merge) + the "
                       "LSE merge of the two states; one_launch: both parts in one mixed launch + one merge pass")
        secondary["shared_prefix_composable"] = leg

    if not args.no_secondary and args.only in ("", "mixed"):
        log("mixed: 64 decode requests + 4 prefill chunks, one mixed launch vs decode + prefill launches")
        secondary["mixed_batch"] = mixed_leg(device, reps=max(10, args.steps // 2))
        torch.cuda.empty_cache()

    if not args.no_secondary and args.only in ("", "ceilings"):
        log("ceilings: bf16 GEMM through torch (vendor BLAS) and a plain device copy, as practical context")
        secondary["practical_ceilings"] = ceilings(device)
        torch.cuda.empty_cache()

    if result:
        result["secondary"] = secondary
        result["kernel_source_hash"] = kernel_source_hash()
        print(json.dumps(result), flush=True)
    else:
        print(json.dumps({"secondary": secondary}), flush=True)


if __name__ == "__main__":
    main()
