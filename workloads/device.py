"""Device copies of a ``workloads.Batch``: q, the physical K/V pools, the page
table and the row counts a RoPE table needs.  Layout plumbing only (no
attention arithmetic); used by the benchmark and by the GPU tests."""
from __future__ import annotations

import numpy as np
import torch

from . import BF16


def torch_dtype(batch):
    return torch.bfloat16 if batch.dtype == BF16 else torch.float32


def upload(batch, layout: str = "HND", device="cuda:0"):
    """Device tensors of a batch: {"q", "k", "v", "pages", "kv_indptr"}.

    Paged: the whole physical pool [num_pages, Hk, page_size, d] ("HND"; "NHD" swaps
    the head and token axes), NaN wherever no live page sits; "pages" is the device
    page table and "kv_indptr" the host page-list offsets.  Dense: [N, Hk, d] blocks,
    "pages" None and "kv_indptr" the host token offsets."""
    dt = torch_dtype(batch)
    dev = torch.device(device)
    out = {"q": torch.from_numpy(batch.q).to(dt).to(dev)}
    if batch.kv_mode == "dense":
        out["k"] = torch.from_numpy(batch.dense_k).to(dt).to(dev)
        out["v"] = torch.from_numpy(batch.dense_v).to(dt).to(dev)
        out["kv_indptr"] = batch.kv_indptr.astype(np.int32)
        out["pages"] = None
        return out
    shape = (batch.num_pages, batch.num_kv_heads, batch.page_size, batch.head_dim)
    k = torch.full(shape, float("nan"), dtype=dt, device=dev)
    v = torch.full(shape, float("nan"), dtype=dt, device=dev)
    phys = torch.from_numpy(batch.kv_page_indices[batch.live_logical].astype(np.int64)).to(dev)
    k[phys] = torch.from_numpy(batch.k_live).to(dt).to(dev)
    v[phys] = torch.from_numpy(batch.v_live).to(dt).to(dev)
    if layout == "NHD":
        k = k.transpose(1, 2).contiguous()
        v = v.transpose(1, 2).contiguous()
    out["k"], out["v"] = k, v
    out["pages"] = torch.from_numpy(batch.kv_page_indices.astype(np.int32)).to(dev)
    out["kv_indptr"] = batch.kv_page_indptr.astype(np.int32)
    return out


def rope_positions_needed(batch) -> int:
    """Rows of the (cos, sin) table a batch's fused-RoPE decode reads: streaming positions are
    ranks in the visible set (at most window + sinks), absolute ones token indices."""
    if batch.rope == "streaming" and batch.window > 0:
        return int(min(int(batch.kv_len.max()), batch.window + batch.sink))
    return int(batch.kv_len.max())
