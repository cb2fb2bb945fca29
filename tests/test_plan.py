"""The C++ planner (through the C ABI, host only) must reproduce the oracle's
reference plan bit for bit: same chunk length, same items in the same order on
every worker, same slots and merge table."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import block_sparse_kv_plan_amd as bsk
import oracle
import workloads as W
from block_sparse_kv_plan_amd.attention import make_problem
from tests import planbuf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def cpp_plan(problem, qo_len, kv_len, kv_indptr=None):
    qo_len = np.asarray(qo_len, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_len)]).astype(np.int32)
    if kv_indptr is None:
        kv_indptr = np.concatenate([[0], np.cumsum((kv_len + 15) // 16)]).astype(np.int32)
    _, _, host_b = bsk.workspace_query(problem)
    host = np.zeros(host_b, dtype=np.uint8)
    info = bsk.plan(problem, qo_indptr, kv_len.astype(np.int32), kv_indptr, host)
    return info, planbuf.decode(host), (qo_indptr, kv_indptr)


KERNEL_MAX_PAGES = 1024  # page ids one item may stage in LDS (documented cap behind max_chunk = 0)


def effective_max_chunk(problem):
    if problem.max_chunk > 0 or problem.kv_mode == bsk.KV_DENSE:
        return problem.max_chunk
    return (KERNEL_MAX_PAGES * problem.page_size) // problem.tile_kv * problem.tile_kv


def ref_params(problem):
    return oracle.PlanParams(
        num_qo_heads=problem.num_qo_heads, num_kv_heads=problem.num_kv_heads, tile_q=problem.tile_q,
        tile_kv=problem.tile_kv, num_workers=problem.num_workers, split_factor=problem.split_factor,
        min_chunk=problem.min_chunk, max_chunk=effective_max_chunk(problem), item_overhead=problem.item_overhead,
        max_items_per_worker=problem.max_items_per_worker, max_slots=problem.max_slots,
        max_merge=problem.max_merge, causal=bool(problem.causal), window=max(problem.window, 0),
        sink=problem.sink if problem.window > 0 else 0, decode_tile_q=problem.decode_tile_q,
        shared_prefix_len=problem.shared_prefix_len)


def assert_same_plan(problem, qo_len, kv_len):
    info, got, (qo_indptr, kv_indptr) = cpp_plan(problem, qo_len, kv_len)
    ref = oracle.plan_ref(qo_len, kv_len, ref_params(problem))
    assert got["chunk"] == ref["chunk"] == info.chunk
    assert got["num_items"] == len(ref["items"]) == info.num_items
    assert got["num_slots"] == ref["num_slots"] == info.num_slots
    assert got["num_merge"] == len(ref["merge"]) == info.num_merge
    for w in range(problem.num_workers):
        ids = ref["worker_items"][w]
        want = np.concatenate([ref["items"][ids], np.asarray(ids, dtype=np.int64)[:, None]], axis=1) \
            if ids else np.zeros((0, 8), dtype=np.int64)
        assert np.array_equal(got["worker_items"][w].astype(np.int64), want), f"worker {w}"
        # the record also carries its request's offsets and lengths, copied from the inputs
        r = got["worker_items"][w][:, 0].astype(np.int64)
        P, T = problem.shared_prefix_len, int(qo_indptr[-1])
        req = np.stack([qo_indptr[r], qo_indptr[r + 1] - qo_indptr[r], np.asarray(kv_len)[r], kv_indptr[r]], axis=1) \
            if len(r) else np.zeros((0, 4), dtype=np.int64)
        if len(r):  # shared-prefix items (r = -1): the batch's global query rows against the dense prefix
            req[r < 0] = [0, T, P, 0]
        assert np.array_equal(got["worker_req"][w].astype(np.int64), req.astype(np.int64)), f"worker {w} request fields"
        assert np.array_equal(got["worker_class"][w].astype(np.int64), ref["item_class"][ids] if ids else
                              np.zeros(0, dtype=np.int64)), f"worker {w} tile classes"
    assert (got["item_pad"] == 0).all()
    assert np.array_equal(got["merge"].astype(np.int64), ref["merge"])
    assert info.max_load == int(ref["load"].max()) if len(ref["items"]) else True
    assert np.array_equal(got["qo_indptr"], qo_indptr)
    assert np.array_equal(got["kv_len"], np.asarray(kv_len, dtype=np.int32))
    assert np.array_equal(got["kv_indptr"], kv_indptr)
    return info, ref


def decode_problem(Hq, Hk, d, W_, dtype=bsk.DTYPE_BF16, **kw):
    return make_problem(num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d, dtype=dtype, num_workers=W_,
                        max_batch=kw.pop("max_batch", 256), **kw)


def test_tiny_decode_matches_golden_and_oracle():
    p = decode_problem(8, 2, 64, 8, dtype=bsk.DTYPE_F32, causal=True, split_factor=2, min_chunk=32,
                       max_chunk=1024, max_items_per_worker=16, max_slots=64, max_merge=64)
    info, ref = assert_same_plan(p, [1, 1, 1, 1], [17, 64, 130, 255])
    assert info.chunk == 64
    assert ref["worker_items"] == [[2, 12], [3, 14], [4, 15], [5, 16], [7, 13], [8, 17], [10, 0, 6], [11, 1, 9]]


def test_llama3_decode_plan():
    qo, kv = W.llama3_decode_lengths()
    p = decode_problem(32, 8, 128, 768, causal=True, max_chunk=4096)
    info, _ = assert_same_plan(p, qo, kv)
    assert info.num_merge > 0


def test_ragged_prefill_plan():
    qo, kv = W.ragged_prefill_lengths()
    p = decode_problem(32, 8, 128, 512, causal=True, tile_q=bsk.TILE_PREFILL, max_chunk=8192)
    assert_same_plan(p, qo, kv)


def test_shared_prefix_plans():
    s = W.shared_prefix_lengths()
    pre = make_problem(num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype=bsk.DTYPE_BF16, kv_mode=bsk.KV_DENSE,
                       tile_q=bsk.TILE_PREFILL, num_workers=512, max_batch=1, max_chunk=4096)
    info, _, _ = cpp_plan(pre, [64], [16384], np.array([0, 16384], dtype=np.int32))
    ref = oracle.plan_ref([64], [16384], ref_params(pre))
    assert info.chunk == ref["chunk"] and info.num_items == len(ref["items"])
    suf = decode_problem(32, 8, 128, 768, causal=True, max_chunk=4096)
    assert_same_plan(suf, np.ones(len(s), dtype=np.int64), s)


def test_streaming_window_plan():
    qo, kv = W.streaming_rope_decode_lengths()
    p = decode_problem(64, 8, 128, 768, causal=True, window=4096, sink=4, max_chunk=4096)
    info, ref = assert_same_plan(p, qo, kv)
    # every unit ends with its sink chunk [0, 4)
    assert all((it[4], it[5]) == (0, 4) for it in ref["items"] if it[5] <= 4)


@pytest.mark.parametrize("seed", range(40))
def test_random_plans(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 20))
    kv = rng.integers(0, 3000, size=B)
    qo = np.minimum(kv, rng.choice([0, 1, 1, 3, 17, 200], size=B))
    Hk = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8]))
    tile_q = int(rng.choice([bsk.TILE_DECODE, bsk.TILE_PREFILL, bsk.TILE_PREFILL_256]))
    window = int(rng.choice([0, 0, 5, 64, 1000]))
    tile_kv = int(rng.choice([16, 32, 64]))
    p = decode_problem(Hk * g, Hk, 64, int(rng.integers(1, 70)), tile_q=tile_q, causal=bool(rng.integers(0, 2)),
                       window=window, sink=int(rng.integers(0, 9)), tile_kv=tile_kv,
                       split_factor=int(rng.integers(1, 5)), min_chunk=tile_kv * int(rng.integers(1, 5)),
                       max_chunk=tile_kv * int(rng.choice([0, 16, 64])) or 0, item_overhead=int(rng.integers(0, 40)),
                       max_items_per_worker=4096, max_slots=1 << 20, max_merge=1 << 20)
    if p.max_chunk and p.max_chunk < p.min_chunk:
        p.max_chunk = p.min_chunk
    if tile_q == bsk.TILE_PREFILL and rng.integers(0, 2):
        p.decode_tile_q = bsk.TILE_DECODE  # mixed launch: two tile classes
    assert_same_plan(p, qo, kv)


def test_mixed_plan_classes():
    """A decode-heavy batch with a few prefill requests: small requests become decode-class items
    (one per kv head and chunk), large ones 128-row items, and the record's class word says which."""
    qo = [1] * 40 + [300, 1, 2, 64, 500] + [1] * 20
    kv = [2000 + 37 * i for i in range(len(qo))]
    kv[40], kv[43], kv[44] = 300, 900, 500
    p = decode_problem(32, 8, 128, 64, tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE, causal=True,
                       split_factor=2, min_chunk=256, max_items_per_worker=4096, max_slots=1 << 20, max_merge=1 << 20)
    info, ref = assert_same_plan(p, qo, kv)
    cls = ref["item_class"]
    assert set(np.unique(cls)) == {0, 1}
    rows = np.asarray(ref["items"])[:, 3] - np.asarray(ref["items"])[:, 2]
    assert rows[cls == 1].max() <= bsk.TILE_DECODE
    assert rows[cls == 0].max() <= bsk.TILE_PREFILL


def composable_problem(W_, P, **kw):
    return decode_problem(32, 8, 128, W_, tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE, causal=True,
                          shared_prefix_len=P, **kw)


def test_composable_one_launch_plan():
    """The shared-prefix workload (16384-token dense prefix, 64 branches with one query token each) as
    one plan: 8 kv heads x 2 prefix tiles of 128 global rows, 512 decode-class suffix units."""
    s = W.shared_prefix_lengths()
    p = composable_problem(512, 16384)
    info, ref = assert_same_plan(p, np.ones(len(s), dtype=np.int64), s)
    cls = ref["item_class"]
    assert set(np.unique(cls)) == {1, 2}
    assert len(ref["merge"]) == 64 * 8 and (ref["merge"][:, 7] > 0).all()
    assert info.num_slots == len(ref["items"])  # every item writes a partial state


@pytest.mark.parametrize("seed", range(24))
def test_random_composable_plans(seed):
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 30))
    kv = rng.integers(1, 3000, size=B)
    qo = np.minimum(kv, rng.choice([1, 1, 1, 2, 3, 4, 5, 40], size=B))  # decode-class and 128-row suffixes
    p = composable_problem(int(rng.integers(1, 90)), int(rng.integers(1, 40000)), tile_kv=64,
                           split_factor=int(rng.integers(1, 4)), min_chunk=64 * int(rng.integers(1, 5)),
                           item_overhead=int(rng.integers(0, 40)), max_items_per_worker=4096, max_slots=1 << 20,
                           max_merge=1 << 20)
    assert_same_plan(p, qo, kv)


def test_composable_requires_the_mixed_launch():
    for kw in (dict(tile_q=bsk.TILE_PREFILL), dict(tile_q=bsk.TILE_PREFILL_256, decode_tile_q=bsk.TILE_DECODE),
               dict(tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE, window=64),
               dict(tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE, fused_merge=1)):
        p = decode_problem(8, 2, 64, 4, shared_prefix_len=100, **kw)
        with pytest.raises(bsk.BskError):
            cpp_plan(p, [1], [10])


def test_mixed_class_requires_prefill_tile_and_paged_kv():
    p = decode_problem(8, 2, 64, 4, tile_q=bsk.TILE_PREFILL_256, decode_tile_q=bsk.TILE_DECODE)
    with pytest.raises(bsk.BskError):
        cpp_plan(p, [1], [10])
    p = decode_problem(8, 2, 64, 4, tile_q=bsk.TILE_PREFILL, decode_tile_q=8)
    with pytest.raises(bsk.BskError):
        cpp_plan(p, [1], [10])
    p = decode_problem(8, 2, 64, 4, tile_q=bsk.TILE_PREFILL, decode_tile_q=bsk.TILE_DECODE, kv_mode=bsk.KV_DENSE)
    with pytest.raises(bsk.BskError):
        cpp_plan(p, [1], [10], kv_indptr=np.array([0, 10], dtype=np.int32))


def test_capacity_and_invalid_errors():
    p = decode_problem(8, 2, 64, 2, max_items_per_worker=4, max_chunk=1024)
    with pytest.raises(bsk.BskError) as e:
        cpp_plan(p, [1] * 40, [100] * 40)
    assert e.value.status == bsk.ERR_CAPACITY
    with pytest.raises(bsk.BskError) as e:
        cpp_plan(p, [5], [3])
    assert e.value.status == bsk.ERR_INVALID_ARG
    p2 = decode_problem(8, 2, 64, 2, max_chunk=1 << 20)
    with pytest.raises(bsk.BskError) as e:
        bsk.workspace_query(p2)
    assert e.value.status == bsk.ERR_INVALID_ARG  # page list would overflow LDS
    p3 = decode_problem(8, 2, 96, 2)
    with pytest.raises(bsk.BskError) as e:
        bsk.workspace_query(p3)
    assert e.value.status == bsk.ERR_UNSUPPORTED


def test_planner_under_host_sanitizers():
    """plan.cpp built with g++ and AddressSanitizer/UBSan, driven over random inputs."""
    drv = os.path.join(ROOT, "tests", "plan_fuzz.cpp")
    src = os.path.join(ROOT, "block_sparse_kv_plan_amd", "csrc", "plan.cpp")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "fuzz")
        subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=all", "-I", os.path.dirname(src), drv, src, "-o", exe])
        out = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=300)
        assert out.returncode == 0, out.stdout + out.stderr
        assert "ok" in out.stdout
