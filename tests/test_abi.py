"""The C-ABI library loads on a machine without a GPU, exports every entry point
include/bsk.h declares, and its ctypes mirrors match the C struct layouts."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import block_sparse_kv_plan_amd as bsk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:bsk_status|const char\*)\s+(bsk_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 18, names
    lib = ctypes.CDLL(bsk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bsk.EXPORTED) == names


def test_status_strings_and_error_path():
    assert bsk.status_string(bsk.ERR_CAPACITY) == "BSK_ERR_CAPACITY"
    p = bsk.Problem()  # zeros: invalid
    with pytest.raises(bsk.BskError) as e:
        bsk.workspace_query(p)
    assert e.value.status == bsk.ERR_INVALID_ARG
    assert "num_qo_heads" in bsk.last_error()


def test_struct_layouts_match_c():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "bsk.h"
#define F(S, m) printf(#S "." #m " %zu\n", offsetof(S, m));
int main(void) {
  printf("bsk_problem %zu\nbsk_plan_info %zu\nbsk_tensors %zu\n", sizeof(bsk_problem), sizeof(bsk_plan_info),
         sizeof(bsk_tensors));
  F(bsk_problem, rope_theta) F(bsk_problem, sm_scale) F(bsk_problem, max_merge) F(bsk_problem, shared_prefix_len)
  F(bsk_plan_info, total_cost) F(bsk_plan_info, used_bytes)
  F(bsk_tensors, kv_page_indices) F(bsk_tensors, lse_stride_tok) F(bsk_tensors, rope_n_pos)
  F(bsk_tensors, prefix_k) F(bsk_tensors, prefix_v_stride_head)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        out = dict(line.split() for line in subprocess.check_output([exe], text=True).splitlines())
    assert int(out["bsk_problem"]) == ctypes.sizeof(bsk.Problem)
    assert int(out["bsk_plan_info"]) == ctypes.sizeof(bsk.PlanInfo)
    assert int(out["bsk_tensors"]) == ctypes.sizeof(bsk.Tensors)
    for key, val in out.items():
        if "." in key:
            s, m = key.split(".")
            cls = {"bsk_problem": bsk.Problem, "bsk_plan_info": bsk.PlanInfo, "bsk_tensors": bsk.Tensors}[s]
            assert getattr(cls, m).offset == int(val), key


def _planned_problem():
    """A decode problem and a host-only plan of it with split units (partial-state slots > 0)."""
    import numpy as np
    from block_sparse_kv_plan_amd.attention import make_problem
    p = make_problem(num_qo_heads=8, num_kv_heads=2, head_dim=128, dtype=bsk.DTYPE_BF16, causal=True, num_workers=4,
                     split_factor=4, min_chunk=64, max_batch=4)
    _, float_b, host_b = bsk.workspace_query(p)
    kv = np.array([900, 300, 77], dtype=np.int32)
    qo = np.array([0, 1, 2, 3], dtype=np.int32)
    ki = np.concatenate([[0], np.cumsum((kv + 15) // 16)]).astype(np.int32)
    info = bsk.plan(p, qo, kv, ki, np.zeros(host_b, dtype=np.uint8))
    assert info.num_slots > 0 and info.num_merge > 0
    t = bsk.Tensors()
    t.q = t.k = t.v = t.out = t.lse = t.kv_page_indices = 0x10000  # never dereferenced: checks come first
    t.q_stride_tok, t.q_stride_head, t.o_stride_tok, t.o_stride_head, t.lse_stride_tok = 8 * 128, 128, 8 * 128, 128, 8
    t.k_stride_page = t.v_stride_page = 2 * 16 * 128
    t.k_stride_head = t.v_stride_head = 16 * 128
    t.k_stride_tok = t.v_stride_tok = 128
    return p, info, t, float_b


def _clone(x):
    return type(x).from_buffer_copy(x)


def _merge_status(p, info, t, int_ws, float_ws, float_bytes):
    import ctypes as C
    return bsk._lib.bsk_merge_states(C.byref(p), C.byref(info), C.byref(t), int_ws, float_ws, float_bytes, None)


def test_merge_states_rejects_bad_workspaces_and_mismatched_plans():
    """bsk_merge_states checks on the host, before anything is enqueued, what the run calls check:
    the float workspace against bsk_workspace_query and the plan against the problem."""
    p, info, t, float_b = _planned_problem()
    fake = 0x20000
    assert _merge_status(p, info, t, fake, None, 0) == bsk.ERR_WORKSPACE
    assert "float workspace" in bsk.last_error()
    assert _merge_status(p, info, t, fake, fake, float_b - 4) == bsk.ERR_WORKSPACE
    bad = _clone(info)
    bad.tile_q = bsk.TILE_PREFILL
    assert _merge_status(p, bad, t, fake, fake, float_b) == bsk.ERR_INVALID_ARG
    assert "query-tile class" in bsk.last_error()
    bad = _clone(info)
    bad.num_workers = info.num_workers + 1
    assert _merge_status(p, bad, t, fake, fake, float_b) == bsk.ERR_INVALID_ARG
    bad = _clone(info)
    bad.num_slots = p.max_slots + 1
    assert _merge_status(p, bad, t, fake, fake, float_b) == bsk.ERR_INVALID_ARG
    assert "capacities" in bsk.last_error()
    bad = _clone(info)
    bad.num_merge = p.max_merge + 1
    assert _merge_status(p, bad, t, fake, fake, float_b) == bsk.ERR_INVALID_ARG
    assert _merge_status(p, info, t, None, fake, float_b) == bsk.ERR_INVALID_ARG
    t2 = _clone(t)
    t2.out = 0x10004  # not 16-byte aligned for f32 out
    assert _merge_status(p, info, t2, fake, fake, float_b) == bsk.ERR_INVALID_ARG


def test_upload_and_merge_upload_reject_bad_arguments():
    """bsk_upload_plan and bsk_merge_states_upload check their arguments on the host before anything
    is enqueued: workspaces against bsk_workspace_query, the plan against its problem and buffers,
    and two distinct int workspaces for the merge and the upload."""
    import ctypes as C
    p, info, t, float_b = _planned_problem()
    int_b, _, host_b = bsk.workspace_query(p)
    fake, fake2, host = 0x20000, 0x40000, 0x80000

    def up(i, hb, iw, ib, hw=host):
        return bsk._lib.bsk_upload_plan(C.byref(p), C.byref(i), hw, hb, iw, ib, None)
    assert up(info, host_b, None, int_b) == bsk.ERR_INVALID_ARG
    assert up(info, host_b, fake, int_b, hw=None) == bsk.ERR_INVALID_ARG
    assert up(info, host_b, fake, int_b - 4) == bsk.ERR_WORKSPACE
    assert up(info, info.used_bytes - 4, fake, int_b) == bsk.ERR_INVALID_ARG
    assert "does not fit" in bsk.last_error()
    for field, value in (("tile_q", bsk.TILE_PREFILL), ("used_bytes", 0), ("used_bytes", info.used_bytes + 2)):
        bad = _clone(info)
        setattr(bad, field, value)
        assert up(bad, host_b, fake, int_b) == bsk.ERR_INVALID_ARG, field

    def mu(iw, fw, fb, nxt, niw, nib):
        return bsk._lib.bsk_merge_states_upload(C.byref(p), C.byref(info), C.byref(t), iw, fw, fb, C.byref(p),
                                                C.byref(nxt), host, host_b, niw, nib, None)
    assert mu(fake, fake, float_b, info, fake, int_b) == bsk.ERR_INVALID_ARG
    assert "another int workspace" in bsk.last_error()
    # distinct pointers whose plan ranges overlap, on either side
    assert info.used_bytes > 256
    for niw in (fake + 256, fake - 256):
        assert mu(fake, fake, float_b, info, niw, int_b) == bsk.ERR_INVALID_ARG
        assert "another int workspace" in bsk.last_error()
    bad = _clone(info)
    bad.used_bytes = 0
    assert bsk._lib.bsk_merge_states_upload(C.byref(p), C.byref(bad), C.byref(t), fake, fake, float_b, C.byref(p),
                                            C.byref(info), host, host_b, fake2, int_b, None) == bsk.ERR_INVALID_ARG
    assert mu(fake, None, 0, info, fake2, int_b) == bsk.ERR_WORKSPACE
    assert mu(fake, fake, float_b - 4, info, fake2, int_b) == bsk.ERR_WORKSPACE
    assert mu(fake, fake, float_b, info, fake2, int_b - 4) == bsk.ERR_WORKSPACE
    assert mu(None, fake, float_b, info, fake2, int_b) == bsk.ERR_INVALID_ARG
    bad = _clone(info)
    bad.num_workers = info.num_workers + 1
    assert mu(fake, fake, float_b, bad, fake2, int_b) == bsk.ERR_INVALID_ARG


def test_run_rejects_the_same_inputs():
    import ctypes as C
    p, info, t, float_b = _planned_problem()
    fake = 0x20000
    run = lambda i, fw, fb: bsk._lib.bsk_run_decode(C.byref(p), C.byref(i), C.byref(t), fake, fw, fb, None)
    assert run(info, fake, float_b - 4) == bsk.ERR_WORKSPACE
    bad = _clone(info)
    bad.num_slots = p.max_slots + 1
    assert run(bad, fake, float_b) == bsk.ERR_INVALID_ARG
    bad = _clone(info)
    bad.num_workers = 3
    assert run(bad, fake, float_b) == bsk.ERR_INVALID_ARG


def test_one_hip_runtime_in_the_process():
    """The library and the binding's host-ordering events use the HIP runtime torch loaded: after
    both are opened only one copy of it is mapped (a second copy would not know torch's streams)."""
    import torch  # noqa: F401
    from block_sparse_kv_plan_amd.attention import _hip_runtime
    _hip_runtime()
    with open("/proc/self/maps") as f:
        mapped = {line.split()[-1] for line in f if "amdhip64" in line}
    assert len(mapped) == 1, mapped


def test_stream_read_rejects_bad_arguments():
    import ctypes as C
    f = bsk._lib.bsk_debug_stream_read
    assert f(None, 1024, 0x10000, 1 << 20, 8, None) == bsk.ERR_INVALID_ARG
    assert f(0x10008, 1024, 0x10000, 1 << 20, 8, None) == bsk.ERR_INVALID_ARG   # src not 16-byte aligned
    assert f(0x10000, 1000, 0x20000, 1 << 20, 8, None) == bsk.ERR_INVALID_ARG   # bytes not a multiple of 16
    assert f(0x10000, 1024, 0x20000, 8 * 256 * 4 - 4, 8, None) == bsk.ERR_INVALID_ARG  # sink too small
    assert f(0x10000, 1024, 0x20000, 1 << 20, 0, None) == bsk.ERR_INVALID_ARG   # empty grid
    assert "grid" in bsk.last_error()


def test_block_read_rejects_bad_arguments():
    f = bsk._lib.bsk_debug_block_read
    ok = dict(src=0x10000, nbytes=1 << 20, order=0x20000, n=16, sink=0x30000, sink_bytes=1 << 20, grid=8)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["src"], a["nbytes"], a["order"], a["n"], a["sink"], a["sink_bytes"], a["grid"], None)
    assert call(src=None) == bsk.ERR_INVALID_ARG
    assert call(order=None) == bsk.ERR_INVALID_ARG
    assert call(sink=None) == bsk.ERR_INVALID_ARG
    assert call(src=0x10008) == bsk.ERR_INVALID_ARG          # not 16-byte aligned
    assert call(nbytes=4096 + 16) == bsk.ERR_INVALID_ARG     # not whole 4 KB blocks
    assert call(nbytes=0) == bsk.ERR_INVALID_ARG
    assert call(order=0x20002) == bsk.ERR_INVALID_ARG        # not int32-aligned
    assert call(n=0) == bsk.ERR_INVALID_ARG
    assert call(grid=0) == bsk.ERR_INVALID_ARG
    assert call(grid=(1 << 20) + 1) == bsk.ERR_INVALID_ARG
    assert call(sink_bytes=8 * 256 * 4 - 4) == bsk.ERR_INVALID_ARG
