"""GPU parity of the unfused RoPE pass (rotated visible keys and query against the oracle's
rotation) and of the unfused pipeline (rotate, then plain decode) against the oracle's reading
of that pipeline (exact rotation, bf16 storage, plain attention) at the stated tolerances."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import oracle
import workloads as W
from block_sparse_kv_plan_amd.attention import BatchAttention, tensors_for
from oracle.attention import PagedKV
from tests.gpu_util import compare, require_gpu, say, upload
from tests.helpers import oracle_kv

pytestmark = pytest.mark.gpu


def _visible(L, window, sink):
    qpos = L - 1
    lo = max(0, qpos - window + 1) if window > 0 else 0
    ns = min(sink, lo) if window > 0 else 0
    return np.concatenate([np.arange(ns), np.arange(lo, L)]).astype(np.int64)


def _ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (for a one-ulp bound on a rounded result)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _rot_bound(x, want):
    """Error bound of a rotation evaluated in fp32 with an fp32 cos/sin table and rounded to bf16:
    one bf16 ulp of the result plus a few fp32 units of the pair's magnitude (x cos - y sin can
    cancel, so the fp32 error is relative to the inputs, not to the result)."""
    half = x.shape[-1] // 2
    pair = np.abs(x[..., :half]) + np.abs(x[..., half:])
    pair = np.concatenate([pair, pair], axis=-1)
    return _ulp_bf16(want) + 4.0 * 2.0 ** -24 * pair


def _setup(b, mode):
    dev = require_gpu()
    du = upload(b)
    n_pos = int(max(b.kv_len))
    rope = torch.empty((n_pos, b.head_dim // 2, 2), dtype=torch.float32, device=dev)
    bsk.rope_table(rope, n_pos, b.head_dim, b.rope_theta, torch.cuda.current_stream())
    rm = {"streaming": bsk.ROPE_STREAMING, "absolute": bsk.ROPE_ABSOLUTE}[mode]
    prob = bsk.attention.make_problem(num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                                      dtype=bsk.DTYPE_BF16, page_size=b.page_size, causal=True, window=b.window,
                                      sink=b.sink, rope_mode=rm, rope_theta=b.rope_theta, num_workers=1,
                                      max_batch=b.batch_size)
    T = int(b.qo_indptr[-1])
    lse = torch.empty((T, b.num_qo_heads), dtype=torch.float32, device=dev)
    out = torch.empty((T, b.num_qo_heads, b.head_dim), dtype=torch.float32, device=dev)
    t = tensors_for(prob, du["q"], du["k"], du["v"], out, lse, page_indices=du["pages"], rope=rope)
    q_out = torch.full_like(du["q"], float("nan"))
    k_out = torch.full_like(du["k"], float("nan"))
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(dev)
    bsk.rope_apply(prob, b.batch_size, int(max(b.kv_len)), i32(b.qo_indptr), i32(b.kv_len), i32(du["kv_indptr"]),
                   t, q_out, q_out.stride(0), q_out.stride(1), k_out, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return du, q_out, k_out, rope


@pytest.mark.parametrize("mode", ["streaming", "absolute"])
def test_rope_apply_matches_oracle_rotation(mode):
    b = W.paged_batch(name=f"rope-apply-{mode}", seed=101, kv_len=[700, 40, 300, 1], qo_len=1, num_qo_heads=8,
                      num_kv_heads=2, head_dim=128, page_size=16, dtype=W.BF16, causal=True, window=256, sink=4,
                      rope=mode, rope_theta=500000.0)
    say(f"rope apply {mode}")
    du, q_out, k_out, _ = _setup(b, mode)
    kp, _ = b.physical_pools()
    got_k = k_out.float().cpu().numpy()
    paged = PagedKV(kp, kp, b.kv_page_indptr, b.kv_page_indices, b.page_size)
    written = np.zeros(got_k.shape[:1] + got_k.shape[2:3], dtype=bool)
    for r in range(b.batch_size):
        L = int(b.kv_len[r])
        vis = _visible(L, b.window, b.sink)
        kpos, qpos = oracle.key_positions(L - 1, vis, mode)
        k_raw, _ = oracle.gather_kv(paged, r, vis)                       # [n, Hk, d]
        want = oracle.rope_rotate(k_raw, kpos[:, None], b.rope_theta)     # fp64
        pages = b.kv_page_indices[b.kv_page_indptr[r] + vis // b.page_size]
        slots = vis % b.page_size
        got = got_k[pages, :, slots, :].astype(np.float64)
        err = np.abs(got - want) - _rot_bound(k_raw, want)
        assert np.all(err <= 0), f"request {r}: worst excess {err.max():.3e}"
        written[pages, slots] = True
        qt = int(b.qo_indptr[r + 1]) - 1
        q_raw = b.q[qt].astype(np.float64)
        wq = oracle.rope_rotate(q_raw, qpos, b.rope_theta)
        gq = q_out[qt].float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(gq - wq) <= _rot_bound(q_raw, wq)), f"query of request {r}"
    # slots of keys no query sees are not written
    untouched = got_k.transpose(0, 2, 1, 3)[~written]
    assert np.isnan(untouched).all()


@pytest.mark.parametrize("mode", ["streaming", "absolute"])
def test_unfused_rope_decode_matches_oracle(mode):
    """Rotate, then a plain windowed decode over (rotated K, V): the RoPE attention result."""
    dev = require_gpu()
    b = W.paged_batch(name=f"rope-unfused-{mode}", seed=102, kv_len=[5000, 40, 4101, 4099, 12000], qo_len=1,
                      num_qo_heads=16, num_kv_heads=2, head_dim=128, page_size=16, dtype=W.BF16, causal=True,
                      window=4096, sink=4, rope=mode, rope_theta=500000.0, poison_invisible=True)
    say(f"unfused rope decode {mode}")
    du, q_out, k_out, _ = _setup(b, mode)
    attn = BatchAttention.create(device=dev, num_qo_heads=16, num_kv_heads=2, head_dim=128, dtype=bsk.DTYPE_BF16,
                                 page_size=16, causal=True, window=4096, sink=4, max_batch=b.batch_size)
    T = int(b.qo_indptr[-1])
    out = torch.empty((T, 16, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((T, 16), dtype=torch.float32, device=dev)
    t = tensors_for(attn.problem, q_out, k_out, du["v"], out, lse, page_indices=du["pages"])
    attn.plan(b.qo_indptr, b.kv_len, du["kv_indptr"])
    attn.run(t)
    torch.cuda.synchronize()
    # The baseline stores the rotated q and k in bf16: the oracle's reading of it rotates in fp64
    # and stores through the same bf16 rounding, so the pipeline is held to the stated bounds.
    ref = oracle.attention_rope_stored(b.q, b.qo_indptr, b.kv_len, oracle_kv(b), b.num_kv_heads, b.sm_scale,
                                       b.window, b.sink, mode, b.rope_theta)
    compare(b, out.double().cpu().numpy(), lse.double().cpu().numpy(), ref=ref)
