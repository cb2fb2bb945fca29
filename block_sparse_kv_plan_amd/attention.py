"""plan/run wrapper over the C ABI, in the shape of a serving engine's batch
attention object: ``plan()`` once per step from host lengths, then ``run()``
(fixed launches, graph-capturable) for every layer.  torch provides device
memory, pinned host memory and streams; all compute is in libbsk's kernels.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import numpy as np
import torch

from . import (DTYPE_BF16, DTYPE_F32, KV_DENSE, KV_PAGED, ROPE_NONE, TILE_DECODE, TILE_PREFILL, TILE_PREFILL_256, PlanInfo,
               Problem, Tensors, append_paged_kv, device_workers, merge_state_pair, merge_states, merge_states_upload,
               plan, run_decode, run_prefill, upload_plan, workspace_query)

TORCH_DTYPE = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}

_HIP_EVENT_DISABLE_TIMING = 0x2
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip = None


def _hip_runtime():
    """The HIP runtime torch has loaded: opened by its soname, which the dynamic loader matches
    against the libraries already in the process (torch's copy), so events and streams share
    one runtime and device state."""
    global _hip
    if _hip is None:
        lib = ctypes.CDLL("libamdhip64.so.7")
        for name in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventSynchronize", "hipEventDestroy"):
            getattr(lib, name).restype = ctypes.c_int
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip = lib
    return _hip


class _HostOrderEvent:
    """A HIP event that only orders the host after GPU work (workspace reuse): created without
    timing and without the system-scope fence, so recording it does not make the queue write back
    its caches for the host, which a torch event does (a few microseconds of GPU time per record).
    Never used to read results on the host or to order another queue."""

    def __init__(self):
        self._lib = _hip_runtime()
        ev = ctypes.c_void_p()
        err = self._lib.hipEventCreateWithFlags(ctypes.byref(ev),
                                                _HIP_EVENT_DISABLE_TIMING | _HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")
        self._ev = ev

    def record(self, stream):
        err = self._lib.hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def synchronize(self):
        err = self._lib.hipEventSynchronize(self._ev)
        if err != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({err})")

    def __del__(self):
        if getattr(self, "_ev", None) is not None and self._lib is not None:
            self._lib.hipEventDestroy(self._ev)

# Plan defaults per query-tile class: (tile_kv, split_factor, min_chunk, max_items_per_worker).
# Decode: one chunk per worker on average; each further item costs a few microseconds of start-up,
# which outweighs the better balance of smaller chunks once the kernel streams near peak.
DEFAULTS = {
    TILE_DECODE: dict(tile_kv=16, split_factor=1, min_chunk=512, max_items_per_worker=64),
    TILE_PREFILL: dict(tile_kv=64, split_factor=1, min_chunk=1024, max_items_per_worker=64),
    TILE_PREFILL_256: dict(tile_kv=64, split_factor=1, min_chunk=1024, max_items_per_worker=64),
}


def make_problem(*, num_qo_heads, num_kv_heads, head_dim, dtype, out_dtype=DTYPE_F32, kv_mode=KV_PAGED,
                 page_size=16, causal=False, window=0, sink=0, rope_mode=ROPE_NONE, rope_theta=10000.0,
                 sm_scale=None, tile_q=TILE_DECODE, num_workers, tile_kv=None, split_factor=None,
                 min_chunk=None, max_chunk=0, item_overhead=0, max_batch, max_items_per_worker=None,
                 max_slots=None, max_merge=None, fused_merge=0, independent_kv_strides=0,
                 decode_tile_q=0, shared_prefix_len=0) -> Problem:
    d = DEFAULTS[tile_q]
    tile_kv = tile_kv if tile_kv is not None else max(d["tile_kv"], page_size if kv_mode == KV_PAGED else 1)
    kmax = max_items_per_worker if max_items_per_worker is not None else d["max_items_per_worker"]
    p = Problem()
    p.num_qo_heads, p.num_kv_heads, p.head_dim = num_qo_heads, num_kv_heads, head_dim
    p.dtype, p.out_dtype, p.kv_mode, p.page_size = dtype, out_dtype, kv_mode, page_size
    p.causal, p.window, p.sink = int(causal), int(window), int(sink)
    p.rope_mode, p.rope_theta = rope_mode, float(rope_theta)
    p.fused_merge = int(fused_merge)
    p.sm_scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim))
    p.tile_q, p.tile_kv, p.num_workers = tile_q, tile_kv, num_workers
    p.split_factor = split_factor if split_factor is not None else d["split_factor"]
    mc = min_chunk if min_chunk is not None else d["min_chunk"]
    p.min_chunk = max(tile_kv, (mc // tile_kv) * tile_kv)
    p.max_chunk, p.item_overhead = max_chunk, item_overhead
    p.max_batch, p.max_items_per_worker = max_batch, kmax
    p.max_slots = max_slots if max_slots is not None else num_workers * kmax
    p.max_merge = max_merge if max_merge is not None else num_workers * kmax
    p.independent_kv_strides = independent_kv_strides
    p.decode_tile_q = decode_tile_q
    p.shared_prefix_len = shared_prefix_len
    return p


def tensors_for(problem: Problem, q, k, v, out, lse, page_indices=None, layout: str = "HND", rope=None,
                prefix_k=None, prefix_v=None) -> Tensors:
    """Describe torch tensors to the C ABI.  PAGED k/v: [pages, Hk, ps, d] ("HND") or
    [pages, ps, Hk, d] ("NHD"); DENSE k/v: [N, Hk, d].  q/out: [T, Hq, d]; lse: [T, Hq].
    prefix_k / prefix_v: the shared dense prefix [P, Hk, d] of a composable batch."""
    t = Tensors()
    t.q, t.q_stride_tok, t.q_stride_head = q.data_ptr(), q.stride(0), q.stride(1)
    t.k, t.v = k.data_ptr(), v.data_ptr()
    if problem.kv_mode == KV_PAGED:
        if layout == "HND":
            t.k_stride_page, t.k_stride_head, t.k_stride_tok = k.stride(0), k.stride(1), k.stride(2)
            t.v_stride_page, t.v_stride_head, t.v_stride_tok = v.stride(0), v.stride(1), v.stride(2)
        elif layout == "NHD":
            t.k_stride_page, t.k_stride_tok, t.k_stride_head = k.stride(0), k.stride(1), k.stride(2)
            t.v_stride_page, t.v_stride_tok, t.v_stride_head = v.stride(0), v.stride(1), v.stride(2)
        else:
            raise ValueError(layout)
        t.kv_page_indices = page_indices.data_ptr()
    else:
        t.k_stride_page, t.k_stride_tok, t.k_stride_head = 0, k.stride(0), k.stride(1)
        t.v_stride_page, t.v_stride_tok, t.v_stride_head = 0, v.stride(0), v.stride(1)
    for x in (q, k, v, out):
        assert x.stride(-1) == 1, "last dimension must be contiguous"
    t.out, t.o_stride_tok, t.o_stride_head = out.data_ptr(), out.stride(0), out.stride(1)
    t.lse, t.lse_stride_tok = lse.data_ptr(), lse.stride(0)
    if rope is not None:
        t.rope_cos_sin, t.rope_n_pos = rope.data_ptr(), rope.shape[0]
    if prefix_k is not None:
        assert prefix_k.stride(-1) == 1 and prefix_v.stride(-1) == 1, "last dimension must be contiguous"
        t.prefix_k, t.prefix_v = prefix_k.data_ptr(), prefix_v.data_ptr()
        t.prefix_k_stride_tok, t.prefix_k_stride_head = prefix_k.stride(0), prefix_k.stride(1)
        t.prefix_v_stride_tok, t.prefix_v_stride_head = prefix_v.stride(0), prefix_v.stride(1)
    return t


class BatchAttention:
    """Owns the workspaces of one problem; plan() per step, run() per layer.

    The plan upload can go on its own copy stream, and the merge can run on a stream of its own
    (merge()): plan() first waits (on the host) for the last run and the last merge that read this
    workspace on other streams, and run() waits (on the GPU) for the upload, so a host plan, its
    copy and the previous step's merge overlap the GPU work already queued.  With two workspaces in
    turn, plan(defer_upload=True) leaves the upload to the other workspace's merge
    (merge(..., upload_next=...)), which then makes it in the same launch."""

    def __init__(self, problem: Problem, device="cuda"):
        self.problem = problem
        int_b, float_b, host_b = workspace_query(problem)
        self.device = torch.device(device)
        self.int_ws = torch.empty(int_b, dtype=torch.uint8, device=self.device)
        self.float_ws = torch.empty(max(float_b, 16), dtype=torch.uint8, device=self.device)
        self.host_ws = torch.empty(host_b, dtype=torch.uint8, pin_memory=True)
        self.info: Optional[PlanInfo] = None
        self._init_order()

    def _init_order(self):
        """The events and streams that order reuse of the workspaces (host and device)."""
        self._uploaded = torch.cuda.Event()   # the plan copy out of host_ws has completed (recorded lazily)
        self._consumed = _HostOrderEvent()    # the last run reading int_ws has completed
        self._merged = _HostOrderEvent()      # the last merge reading int_ws / float_ws has completed
        self._consumed_stream = None
        self._merged_stream = None
        self._run_stream = None  # stream of a run(merge=False) whose merge() has not been called yet
        self._upload_pending = False
        self._upload_stream = None
        # An event recorded on the kernels' queue costs GPU time (it ends in a release the host can
        # see), so the upload gets one only when something needs it: a run on another stream, or
        # the next plan when no run of this plan has been merged or settled since.  Every run waits
        # for its plan's upload, so the event of its merge (or its own, when the merge is fused or
        # never called) completes after the upload too, and the next plan waits for that instead:
        # an upload event recorded only then would sit behind all the work queued meanwhile.
        self._upload_recorded = False
        self._ran = False          # a run (or replay) of the last plan has been launched
        self._upload_cover = None  # an event recorded after such a run, hence after the upload
        self._deferred = None      # the stream a deferred upload of the last plan must go to

    @classmethod
    def create(cls, *, device="cuda", num_workers=None, **kw):
        if num_workers is None:
            num_workers = device_workers(make_problem(num_workers=1, **kw))
        return cls(make_problem(num_workers=num_workers, **kw), device=device)

    def _record_upload(self):
        if not self._upload_recorded:
            self._uploaded.record(self._upload_stream)
            self._upload_recorded = True

    def _recorded(self, ev):
        """Note that `ev` has just been recorded after a run of the last plan (a run waits for its
        plan's upload, and a merge on another stream waits for the run), so it completes after
        the upload."""
        if self._upload_pending and self._ran:
            self._upload_cover = ev

    def plan(self, qo_indptr, kv_len, kv_indptr, stream=None, copy_stream=None, defer_upload=False) -> PlanInfo:
        """Plan the step on the host and upload it (on copy_stream if given, else on `stream`).  With
        defer_upload the upload is left to upload() or to another workspace's merge(upload_next=...),
        on that same stream; until then run() refuses to start."""
        self._deferred = None  # a deferred upload not made yet is superseded: nothing of it is queued
        self._settle_run()
        synced = None
        if self._upload_pending:  # host_ws may still be read by the previous upload
            if self._upload_cover is not None:
                synced = self._upload_cover
            else:
                self._record_upload()
                synced = self._uploaded
            synced.synchronize()
        stream = stream or torch.cuda.current_stream(self.device)
        up = copy_stream if copy_stream is not None else stream
        # Do not overwrite int_ws under a kernel that still reads it on another stream: wait for the
        # last run and the last merge (one wait when both went to the same stream, the merge last).
        # The wait is on the host.  A GPU-side wait queued in front of the upload made every copy
        # behind it cost ~50 us of host time in the runtime, and once per process stalled one copy
        # for several milliseconds; with two or more workspaces in turn the last run on this one
        # has normally finished by the time it is planned again, so the host wait returns at once.
        # (a torch stream compares unequal to nothing, None included: `stream != None` is False)
        waits = []
        if self._merged_stream is not None:
            waits.append((self._merged, self._merged_stream))
        if self._consumed_stream is not None and (self._merged_stream is None
                                                  or self._consumed_stream != self._merged_stream):
            waits.append((self._consumed, self._consumed_stream))
        for ev, st in waits:
            if st != up and ev is not synced:
                ev.synchronize()
        if defer_upload:
            self.info = plan(self.problem, np.asarray(qo_indptr), np.asarray(kv_len), np.asarray(kv_indptr),
                             self.host_ws)
            self._upload_pending = False  # nothing queued reads host_ws until the upload is made
            self._deferred = up
            self._ran = False
            self._upload_cover = None
            return self.info
        self.info = plan(self.problem, np.asarray(qo_indptr), np.asarray(kv_len), np.asarray(kv_indptr),
                         self.host_ws, self.int_ws, up)
        self._uploaded_on(up)
        return self.info

    def _uploaded_on(self, stream):
        """The last plan's upload has just been enqueued on `stream`."""
        self._deferred = None
        self._upload_pending = True
        self._upload_stream = stream
        self._upload_recorded = False
        self._ran = False
        self._upload_cover = None

    def _deferred_stream(self, stream):
        if self._deferred is None:
            raise RuntimeError("no deferred upload: plan(..., defer_upload=True) first")
        stream = stream or self._deferred
        if stream != self._deferred:
            raise ValueError("a deferred upload goes to the stream its plan named (its reuse waits were taken for it)")
        return stream

    def upload(self, stream=None):
        """Make the deferred upload of the last plan on `stream` (the stream the plan named)."""
        stream = self._deferred_stream(stream)
        upload_plan(self.problem, self.info, self.host_ws, self.int_ws, stream)
        self._uploaded_on(stream)

    def _refuse_deferred(self):
        if self._deferred is not None:
            raise RuntimeError("the last plan's upload is deferred: upload() it, or merge another workspace's run "
                               "with upload_next=this workspace, first")

    def run(self, tensors: Tensors, stream=None, merge: bool = True, wait_upload: bool = True):
        """Attention (and, unless merge is False, the merge) for the last plan.  A plan uploaded on
        another stream is waited for on `stream` first; wait_upload=False leaves that wait to the
        caller (who must have made `stream` wait for the upload already)."""
        self._refuse_deferred()
        stream = stream or torch.cuda.current_stream(self.device)
        if wait_upload and self._upload_stream is not None and self._upload_stream != stream:
            self._record_upload()
            stream.wait_event(self._uploaded)
        if self.problem.tile_q == TILE_DECODE:
            run_decode(self.problem, self.info, tensors, self.int_ws, self.float_ws, stream)
        else:
            run_prefill(self.problem, self.info, tensors, self.int_ws, self.float_ws, stream)
        self._ran = True
        self._consumed_stream = None
        self._merged_stream = None  # the last merge event belongs to an earlier run
        # The merge that follows (on this stream, or on one the caller made wait for this run) ends
        # after the run, so its event also covers the run; the run's own event -- a packet on the
        # queue that costs microseconds -- is recorded only if no merge comes (_settle_run).
        self._run_stream = stream
        if merge:
            self.merge(tensors, stream)

    def _settle_run(self):
        """Record the consumed event of a run whose merge was never called (conservatively: after
        everything queued on the run's stream so far)."""
        if self._run_stream is not None:
            self._consumed.record(self._run_stream)
            self._recorded(self._consumed)
            self._consumed_stream = self._run_stream
            self._run_stream = None

    def capture(self, tensors: Tensors, stream=None) -> "torch.cuda.CUDAGraph":
        """Record this workspace's run (and merge, unless it is fused) for `tensors` in a graph.

        The run and merge launches read every per-step value from the int workspace (FlashInfer
        paper summary, "Research methodology" 3: a plan cached on the GPU drives a fixed launch),
        so one capture serves every later plan into the same workspace; replay() runs it after
        each plan().  `stream` is the capturing stream (a side stream is made if none is given)."""
        stream = stream or torch.cuda.Stream(self.device)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            if self.problem.tile_q == TILE_DECODE:
                run_decode(self.problem, self.info, tensors, self.int_ws, self.float_ws, stream)
            else:
                run_prefill(self.problem, self.info, tensors, self.int_ws, self.float_ws, stream)
            if not self.problem.fused_merge:
                merge_states(self.problem, self.info, tensors, self.int_ws, self.float_ws, stream)
        return graph

    def replay(self, graph: "torch.cuda.CUDAGraph", stream=None):
        """Run a graph from capture() on `stream` for the last plan: waits for the plan's upload
        when it went to another stream, and counts as the run and merge of this workspace for the
        next plan's reuse checks."""
        self._refuse_deferred()
        stream = stream or torch.cuda.current_stream(self.device)
        if self._upload_stream is not None and self._upload_stream != stream:
            self._record_upload()
            stream.wait_event(self._uploaded)
        with torch.cuda.stream(stream):
            graph.replay()
        self._ran = True
        self._merged.record(stream)
        self._recorded(self._merged)
        self._merged_stream = stream
        self._consumed_stream = None
        self._run_stream = None

    def merge(self, tensors: Tensors, stream=None, upload_next: Optional["BatchAttention"] = None):
        """The split-KV merge of the last run (nothing when the run merged in-kernel).  On another
        stream than the run's, the caller makes that stream wait for the run first.  upload_next:
        another workspace whose last plan was made with defer_upload=True for this stream; its
        upload goes in the same launch as the merge."""
        stream = stream or torch.cuda.current_stream(self.device)
        if upload_next is not None:
            if upload_next is self:
                raise ValueError("upload_next must be another workspace")
            upload_next._deferred_stream(stream)
        if self.problem.fused_merge:
            self._settle_run()
            if upload_next is not None:
                upload_next.upload(stream)
            return
        if upload_next is None:
            merge_states(self.problem, self.info, tensors, self.int_ws, self.float_ws, stream)
        else:
            merge_states_upload(self.problem, self.info, tensors, self.int_ws, self.float_ws, upload_next.problem,
                                upload_next.info, upload_next.host_ws, upload_next.int_ws, stream)
            upload_next._uploaded_on(stream)
        self._merged.record(stream)
        self._recorded(self._merged)
        self._merged_stream = stream
        self._run_stream = None


def merge_pair(o_a, lse_a, o_b, lse_b, o_out, lse_out, stream=None):
    """Row-wise state merge of two complete (O f32 [..., d], LSE f32 [...]) states."""
    rows = lse_a.numel()
    d = o_a.shape[-1]
    out_dtype = DTYPE_BF16 if o_out.dtype == torch.bfloat16 else DTYPE_F32
    merge_state_pair(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, d, out_dtype,
                     stream or torch.cuda.current_stream(o_a.device))


def run_composable(prefix: BatchAttention, prefix_tensors: Tensors, prefix_state, suffix: BatchAttention,
                   suffix_tensors: Tensors, suffix_state, out, lse, stream=None, side_stream=None):
    """Composable format (FlashInfer paper summary, "Research methodology" 1): attention over a
    dense shared prefix and over each request's paged suffix, each with its own kernel and block
    size, then the two states merged by LSE into (out, lse).

    Both parts must already be planned; each run writes its own state into the (O f32, LSE) pair
    its tensors name, passed again as prefix_state / suffix_state for the merge.  With a side stream the suffix runs there while the prefix runs on
    `stream` -- the prefix is MFMA-bound and the suffix HBM-bound, so the two overlap when each
    plan was made for part of the GPU (num_workers below bsk_device_workers) -- and `stream` waits
    for the side stream before the merge.  Without one, the three steps run in order on `stream`.
    Both orders give identical results (the plans fix every partial state and merge)."""
    stream = stream or torch.cuda.current_stream(out.device)
    if side_stream is not None:
        start = torch.cuda.Event()
        start.record(stream)
        side_stream.wait_event(start)
        suffix.run(suffix_tensors, stream=side_stream)
        prefix.run(prefix_tensors, stream=stream)
        done = torch.cuda.Event()
        done.record(side_stream)
        stream.wait_event(done)
    else:
        prefix.run(prefix_tensors, stream=stream)
        suffix.run(suffix_tensors, stream=stream)
    merge_pair(prefix_state[0], prefix_state[1], suffix_state[0], suffix_state[1], out, lse, stream)


def pool_strides(pool, layout="HND"):
    """(page, head, token) element strides of a K or V pool tensor."""
    if layout == "HND":
        return pool.stride(0), pool.stride(1), pool.stride(2)
    if layout == "NHD":
        return pool.stride(0), pool.stride(2), pool.stride(1)
    raise ValueError(layout)


def chunked_prefill(attn: BatchAttention, q, k_new, v_new, out, lse, k_pool, v_pool, page_indices,
                    kv_page_indptr, prefix_len, new_len, chunk_tokens: int, layout="HND", stream=None):
    """Causal prefill of new tokens appended after cached ones, in steps of at most chunk_tokens
    tokens (chunked prefill, FlashInfer 0.6 wiki "Kernel types": Prefill).

    The new tokens are the rows of q / k_new / v_new, request after request (new_len[r] rows of
    request r, whose first prefix_len[r] tokens are already in the cache).  Step s takes rows
    [s * chunk_tokens, (s + 1) * chunk_tokens): each request contributes one contiguous run of its
    tokens, so the step's q, K/V and output rows are views.  A step appends its rows' K/V to the
    pages (bsk_append_paged_kv), plans the step with kv_len = cached + appended so far, and runs
    the prefill kernel plus the merge; all device work is the library's.  attn must be a
    prefill-class BatchAttention over the same problem; kv_page_indptr is a host array."""
    stream = stream or torch.cuda.current_stream(attn.device)
    prefix_len = np.asarray(prefix_len, dtype=np.int64)
    new_len = np.asarray(new_len, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(new_len)])
    n_total = int(starts[-1])
    page_indptr_host = np.asarray(kv_page_indptr, dtype=np.int32)
    ks, vs = pool_strides(k_pool, layout), pool_strides(v_pool, layout)
    p = attn.problem
    # The device index arrays are allocated while `stream` is current: the caching allocator then
    # hands their blocks only to later allocations on `stream`, which run after the appends that
    # read them, so a caller's stream other than the current one is safe.
    steps = []
    for c0 in range(0, n_total, chunk_tokens):
        c1 = min(c0 + chunk_tokens, n_total)
        lo = np.clip(c0 - starts[:-1], 0, new_len)
        hi = np.clip(c1 - starts[:-1], 0, new_len)
        qo_indptr = np.concatenate([[0], np.cumsum(hi - lo)]).astype(np.int32)
        kv_len = (prefix_len + hi).astype(np.int32)
        steps.append((c0, c1, qo_indptr, kv_len))
    with torch.cuda.stream(stream):
        page_indptr_dev = torch.as_tensor(page_indptr_host).to(attn.device)
        dev = [(torch.as_tensor(qo).to(attn.device), torch.as_tensor(kl).to(attn.device)) for _, _, qo, kl in steps]
    for (c0, c1, qo_indptr, kv_len), (app_dev, kvl_dev) in zip(steps, dev):
        kn, vn = k_new[c0:c1], v_new[c0:c1]
        append_paged_kv(p, len(new_len), c1 - c0, app_dev, kvl_dev, page_indptr_dev, page_indices, kn, vn,
                        kn.stride(0), kn.stride(1), k_pool, v_pool, ks, vs, stream)
        attn.plan(qo_indptr, kv_len, page_indptr_host, stream=stream)
        t = tensors_for(p, q[c0:c1], k_pool, v_pool, out[c0:c1], lse[c0:c1], page_indices=page_indices,
                        layout=layout)
        attn.run(t, stream=stream)
