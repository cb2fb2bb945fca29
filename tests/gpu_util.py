"""GPU test helpers: upload a workloads.Batch, run it through the C ABI, compare
with the oracle.  Test infrastructure only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_kv_plan_amd as bsk
from block_sparse_kv_plan_amd.attention import BatchAttention, make_problem, tensors_for
from tests.helpers import oracle_attention
from workloads.device import rope_positions_needed, torch_dtype, upload  # noqa: F401 (re-exported)

O_TOL = 1e-2    # max-abs on O: bf16 inputs, fp32 accumulation
LSE_TOL = 1e-3  # max-abs on LSE


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def tdtype(batch):
    return torch_dtype(batch)


def run(batch, tile_q=bsk.TILE_DECODE, out_dtype=bsk.DTYPE_F32, layout="HND", dev_tensors=None, num_workers=None,
        stream=None, **plan_kw):
    """Plan + run + merge through the C ABI; returns (O float64 [T,Hq,d], LSE float64 [T,Hq], attn, tensors)."""
    device = require_gpu()
    d = dev_tensors if dev_tensors is not None else upload(batch, layout)
    rope_mode = {"none": bsk.ROPE_NONE, "streaming": bsk.ROPE_STREAMING, "absolute": bsk.ROPE_ABSOLUTE}[batch.rope]
    kw = dict(num_qo_heads=batch.num_qo_heads, num_kv_heads=batch.num_kv_heads, head_dim=batch.head_dim,
              dtype=bsk.DTYPE_BF16 if batch.dtype == "bf16" else bsk.DTYPE_F32, out_dtype=out_dtype,
              kv_mode=bsk.KV_DENSE if batch.kv_mode == "dense" else bsk.KV_PAGED,
              page_size=batch.page_size if batch.kv_mode == "paged" else 16, causal=batch.causal,
              window=batch.window, sink=batch.sink, rope_mode=rope_mode, rope_theta=batch.rope_theta,
              sm_scale=batch.sm_scale, tile_q=tile_q, max_batch=max(1, batch.batch_size))
    kw.update(plan_kw)
    attn = BatchAttention.create(device=device, num_workers=num_workers, **kw)
    T = int(batch.qo_indptr[-1])
    o_dt = torch.bfloat16 if out_dtype == bsk.DTYPE_BF16 else torch.float32
    out = torch.full((T, batch.num_qo_heads, batch.head_dim), float("nan"), dtype=o_dt, device=device)
    lse = torch.full((T, batch.num_qo_heads), float("nan"), dtype=torch.float32, device=device)
    rope = None
    if rope_mode != bsk.ROPE_NONE:
        n_pos = rope_positions_needed(batch)
        rope = torch.empty((n_pos, batch.head_dim // 2, 2), dtype=torch.float32, device=device)
        bsk.rope_table(rope, n_pos, batch.head_dim, batch.rope_theta, torch.cuda.current_stream())
    t = tensors_for(attn.problem, d["q"], d["k"], d["v"], out, lse, page_indices=d["pages"], layout=layout,
                    rope=rope)
    attn.plan(batch.qo_indptr, batch.kv_len, d["kv_indptr"], stream=stream)
    attn.run(t, stream=stream)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), attn, (t, out, lse, d, rope)


def compare(batch, O, L, tokens=None, o_tol=O_TOL, lse_tol=LSE_TOL, ref=None, out_bf16=False):
    """Oracle comparison on all tokens (or a sample); returns (max|dO|, max|dLSE|).  out_bf16: O was
    written in bf16, i.e. the fp32 result rounded to nearest even, so each element may also carry
    that rounding: at most 2^-8 of its magnitude on top of o_tol."""
    Oref, Lref = ref if ref is not None else oracle_attention(batch, tokens=tokens)
    sel = slice(None) if tokens is None else np.asarray(tokens)
    do = np.abs(O[sel] - Oref[sel])
    dl = np.abs(L[sel] - Lref[sel])
    assert np.isfinite(O[sel]).all() and np.isfinite(L[sel]).all(), "non-finite output"
    eo, el = float(do.max()), float(dl.max())
    say(f"  {batch.name}: max|dO| = {eo:.3e}  max|dLSE| = {el:.3e}")
    if out_bf16:
        bound = o_tol + (np.abs(Oref[sel]) + o_tol) * 2.0 ** -8
        worst = float((do - bound).max())
        assert worst <= 0, f"O error beyond the bf16 output bound by {worst}"
    else:
        assert eo <= o_tol, f"O error {eo}"
    assert el <= lse_tol, f"LSE error {el}"
    return eo, el
