"""GPU parity of the K/V append (bit-exact against the oracle) and of chunked prefill built on it
(against the oracle's prefill of the whole sequence)."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
import oracle
import workloads as W
from block_sparse_kv_plan_amd.attention import BatchAttention, chunked_prefill, pool_strides
from oracle.attention import PagedKV
from tests.gpu_util import compare, require_gpu, say

pytestmark = pytest.mark.gpu


def _bits(x):
    """Bit pattern view (NaN-safe equality)."""
    x = np.ascontiguousarray(x)
    return x.view(np.uint16 if x.dtype.itemsize == 2 else np.uint32)


def _case(seed, prefix, new, Hk, d, ps, dtype, layout, kv_len_after=None):
    rng = np.random.default_rng(seed)
    prefix = np.asarray(prefix, dtype=np.int64)
    new = np.asarray(new, dtype=np.int64)
    after = prefix + new if kv_len_after is None else np.asarray(kv_len_after, dtype=np.int64)
    pages = (np.maximum(after, prefix + new) + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    pool = int(indptr[-1]) + 5
    perm = rng.permutation(pool)[:int(indptr[-1])].astype(np.int32)
    shape = (pool, Hk, ps, d) if layout == "HND" else (pool, ps, Hk, d)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    k[rng.random(shape) < 0.05] = np.nan  # poison: untouched slots must keep their exact bits
    app = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    kn = rng.standard_normal((int(app[-1]), Hk, d)).astype(np.float32)
    vn = rng.standard_normal((int(app[-1]), Hk, d)).astype(np.float32)
    if dtype == W.BF16:
        k, v, kn, vn = (W.round_bf16(x) for x in (k, v, kn, vn))
    return dict(k=k, v=v, indptr=indptr, perm=perm, app=app, after=after.astype(np.int32), kn=kn, vn=vn)


@pytest.mark.parametrize("dtype,d,ps,layout", [(W.BF16, 128, 16, "HND"), (W.BF16, 64, 1, "HND"),
                                               (W.F32, 64, 8, "HND"), (W.F32, 128, 32, "NHD"),
                                               (W.BF16, 128, 64, "NHD")])
def test_append_bit_exact(dtype, d, ps, layout):
    dev = require_gpu()
    Hk = 4
    c = _case(80 + ps, prefix=[5, 0, 37, 16, 3], new=[3, 21, 0, 16, 40], Hk=Hk, d=d, ps=ps, dtype=dtype,
              layout=layout)
    say(f"append {dtype} d={d} ps={ps} {layout}")
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    kp = torch.from_numpy(c["k"]).to(tdt).to(dev)
    vp = torch.from_numpy(c["v"]).to(tdt).to(dev)
    kn = torch.from_numpy(c["kn"]).to(tdt).to(dev)
    vn = torch.from_numpy(c["vn"]).to(tdt).to(dev)
    prob = bsk.attention.make_problem(num_qo_heads=Hk, num_kv_heads=Hk, head_dim=d,
                                      dtype=bsk.DTYPE_BF16 if dtype == W.BF16 else bsk.DTYPE_F32, page_size=ps,
                                      num_workers=1, max_batch=8)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(dev)
    bsk.append_paged_kv(prob, len(c["after"]), int(c["app"][-1]), t(c["app"]), t(c["after"]), t(c["indptr"]),
                        t(c["perm"]), kn, vn, kn.stride(0), kn.stride(1), kp, vp, pool_strides(kp, layout),
                        pool_strides(vp, layout), torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.append_paged_kv(c["k"], c["v"], c["indptr"], c["perm"], ps, c["app"], c["after"],
                                          c["kn"], c["vn"], layout=layout)
    got_k = kp.cpu().numpy() if dtype == W.F32 else kp.view(torch.int16).cpu().numpy()
    got_v = vp.cpu().numpy() if dtype == W.F32 else vp.view(torch.int16).cpu().numpy()
    if dtype == W.BF16:
        want_k = torch.from_numpy(ref_k).to(torch.bfloat16).view(torch.int16).numpy()
        want_v = torch.from_numpy(ref_v).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)
    else:
        assert np.array_equal(_bits(got_k), _bits(ref_k)) and np.array_equal(_bits(got_v), _bits(ref_v))


def test_append_skips_positions_outside_the_page_list():
    """kv_len shorter than the new tokens (negative positions) and positions past the page list
    write nothing: the pools keep every bit."""
    dev = require_gpu()
    c = _case(90, prefix=[4, 2], new=[6, 3], Hk=2, d=64, ps=4, dtype=W.F32, layout="HND", kv_len_after=[3, 5])
    indptr = c["indptr"].copy()
    indptr[1:] = np.minimum(indptr[1:], indptr[:-1] + 1)  # request 0 keeps one page of its list
    kp = torch.from_numpy(c["k"]).to(dev)
    vp = torch.from_numpy(c["v"]).to(dev)
    kn = torch.from_numpy(c["kn"]).to(dev)
    vn = torch.from_numpy(c["vn"]).to(dev)
    prob = bsk.attention.make_problem(num_qo_heads=2, num_kv_heads=2, head_dim=64, dtype=bsk.DTYPE_F32,
                                      page_size=4, num_workers=1, max_batch=8)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(dev)
    bsk.append_paged_kv(prob, 2, int(c["app"][-1]), t(c["app"]), t(c["after"]), t(indptr), t(c["perm"]), kn, vn,
                        kn.stride(0), kn.stride(1), kp, vp, pool_strides(kp), pool_strides(vp),
                        torch.cuda.current_stream())
    torch.cuda.synchronize()
    # request 0: kv_len 3 < 6 new tokens -> positions -3..2; 0..2 in page 0 are written, the rest skipped;
    # request 1: positions 2..4, all inside its (shifted) page list
    ref_k, ref_v = c["k"].copy(), c["v"].copy()
    for r, positions in ((0, range(-3, 3)), (1, range(2, 5))):
        for i, pos in enumerate(positions):
            if pos < 0 or pos // 4 >= indptr[r + 1] - indptr[r]:
                continue
            page = c["perm"][indptr[r] + pos // 4]
            ref_k[page, :, pos % 4] = c["kn"][c["app"][r] + i]
            ref_v[page, :, pos % 4] = c["vn"][c["app"][r] + i]
    assert np.array_equal(_bits(kp.cpu().numpy()), _bits(ref_k))
    assert np.array_equal(_bits(vp.cpu().numpy()), _bits(ref_v))


@pytest.mark.parametrize("tile_q,chunk", [(bsk.TILE_PREFILL, 300), (bsk.TILE_PREFILL, 1000),
                                          (bsk.TILE_PREFILL_256, 777)])
def test_chunked_prefill_matches_whole_prefill(tile_q, chunk):
    """Ragged prefill with append, run as chunk steps (append, then attend over cached + appended),
    equals the oracle's prefill of the whole sequence."""
    dev = require_gpu()
    prefix = np.array([0, 300, 1024, 17, 0, 640])
    new = np.array([700, 129, 1, 900, 64, 333])
    b = W.paged_batch(name=f"chunked-{chunk}", seed=95, kv_len=prefix + new, qo_len=new, num_qo_heads=16,
                      num_kv_heads=4, head_dim=128, page_size=16, dtype=W.BF16, causal=True)
    say(f"chunked prefill tile_q={tile_q} chunk={chunk}: {int(new.sum())} new tokens")
    from tests.gpu_util import upload
    du = upload(b)
    kp, vp = du["k"], du["v"]
    # the new tokens' K/V as the model would produce them, taken from the full sequence; their
    # slots in the pools are then cleared, so the result depends on the appends
    phys = PagedKV(*b.physical_pools(), b.kv_page_indptr, b.kv_page_indices, b.page_size)
    ks, vs, pg, sl = [], [], [], []
    for r in range(b.batch_size):
        pos = np.arange(prefix[r], prefix[r] + new[r])
        kk, vv = oracle.gather_kv(phys, r, pos)
        ks.append(kk)
        vs.append(vv)
        pg.append(b.kv_page_indices[b.kv_page_indptr[r] + pos // 16])
        sl.append(pos % 16)
    kn = torch.from_numpy(np.concatenate(ks).astype(np.float32)).to(torch.bfloat16).to(dev)
    vn = torch.from_numpy(np.concatenate(vs).astype(np.float32)).to(torch.bfloat16).to(dev)
    pg_t = torch.from_numpy(np.concatenate(pg).astype(np.int64)).to(dev)
    sl_t = torch.from_numpy(np.concatenate(sl).astype(np.int64)).to(dev)
    kp[pg_t, :, sl_t] = float("nan")
    vp[pg_t, :, sl_t] = float("nan")
    attn = BatchAttention.create(device=dev, num_qo_heads=16, num_kv_heads=4, head_dim=128, dtype=bsk.DTYPE_BF16,
                                 page_size=16, causal=True, tile_q=tile_q, max_batch=b.batch_size)
    T = int(new.sum())
    out = torch.full((T, 16, 128), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((T, 16), float("nan"), dtype=torch.float32, device=dev)
    chunked_prefill(attn, du["q"], kn, vn, out, lse, kp, vp, du["pages"], du["kv_indptr"], prefix, new, chunk)
    torch.cuda.synchronize()
    compare(b, out.double().cpu().numpy(), lse.double().cpu().numpy())
