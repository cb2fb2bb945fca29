"""Python binding of libbsk (include/bsk.h): argument marshalling only.

Every function here has the name of its C entry point without the ``bsk_``
prefix and forwards to it through ctypes; all attention work runs in the
HIP kernels of libbsk.so.  Pointers may be given as ints or as objects
with ``data_ptr()`` (torch tensors); host arrays as numpy int32 arrays.
Importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# torch ships its own HIP/HSA runtime under the same sonames as /opt/rocm's.  Importing it first
# makes libbsk's libamdhip64.so.7 / libhsa-runtime64.so.1 resolve to those already-loaded copies,
# so the process holds one runtime and torch tensors and libbsk kernels share the device.  Loading
# libbsk first would bring in a second runtime that does not see the device torch has opened.
import torch  # noqa: F401  (load order only)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsk.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python block_sparse_kv_plan_amd/build.py` "
                      "(or __graft_entry__.build()) -- there is no fallback path")
_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20  # BSK_NOALLOC_SCRATCH_BYTES
DTYPE_F32, DTYPE_BF16 = 0, 1
KV_PAGED, KV_DENSE = 0, 1
ROPE_NONE, ROPE_STREAMING, ROPE_ABSOLUTE = 0, 1, 2
TILE_DECODE, TILE_PREFILL, TILE_PREFILL_256 = 16, 128, 256

i32, i64, f32, f64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class Problem(ctypes.Structure):
    _fields_ = [("num_qo_heads", i32), ("num_kv_heads", i32), ("head_dim", i32), ("dtype", i32),
                ("out_dtype", i32), ("kv_mode", i32), ("page_size", i32), ("causal", i32), ("window", i32),
                ("sink", i32), ("rope_mode", i32), ("fused_merge", i32), ("rope_theta", f64), ("sm_scale", f32),
                ("tile_q", i32), ("tile_kv", i32), ("num_workers", i32), ("split_factor", i32),
                ("min_chunk", i32), ("max_chunk", i32), ("item_overhead", i32), ("max_batch", i32),
                ("max_items_per_worker", i32), ("max_slots", i32), ("max_merge", i32),
                ("independent_kv_strides", i32), ("decode_tile_q", i32), ("shared_prefix_len", i32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_workers", i32), ("tile_q", i32), ("batch", i32), ("num_items", i32), ("num_slots", i32),
                ("num_merge", i32), ("chunk", i32), ("max_kv_len", i32), ("max_qo_len", i32),
                ("max_items_on_worker", i32), ("total_cost", i64), ("max_load", i64), ("used_bytes", i64)]


class Tensors(ctypes.Structure):
    _fields_ = [("q", vp), ("q_stride_tok", i64), ("q_stride_head", i64), ("k", vp), ("v", vp),
                ("k_stride_page", i64), ("k_stride_head", i64), ("k_stride_tok", i64),
                ("v_stride_page", i64), ("v_stride_head", i64), ("v_stride_tok", i64),
                ("kv_page_indices", vp), ("out", vp), ("o_stride_tok", i64), ("o_stride_head", i64),
                ("lse", vp), ("lse_stride_tok", i64), ("rope_cos_sin", vp), ("rope_n_pos", i32),
                ("reserved0", i32), ("prefix_k", vp), ("prefix_v", vp), ("prefix_k_stride_tok", i64),
                ("prefix_k_stride_head", i64), ("prefix_v_stride_tok", i64), ("prefix_v_stride_head", i64)]


P = ctypes.POINTER
_lib.bsk_status_string.restype = ctypes.c_char_p
_lib.bsk_status_string.argtypes = [i32]
_lib.bsk_last_error.restype = ctypes.c_char_p
_lib.bsk_last_error.argtypes = []
_sig = {
    "bsk_device_workers": [P(Problem), P(i32)],
    "bsk_workspace_query": [P(Problem), P(ctypes.c_size_t), P(ctypes.c_size_t), P(ctypes.c_size_t)],
    "bsk_plan": [P(Problem), i32, vp, vp, vp, vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp, P(PlanInfo)],
    "bsk_run_decode": [P(Problem), P(PlanInfo), P(Tensors), vp, vp, ctypes.c_size_t, vp],
    "bsk_run_prefill": [P(Problem), P(PlanInfo), P(Tensors), vp, vp, ctypes.c_size_t, vp],
    "bsk_upload_plan": [P(Problem), P(PlanInfo), vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp],
    "bsk_merge_states": [P(Problem), P(PlanInfo), P(Tensors), vp, vp, ctypes.c_size_t, vp],
    "bsk_merge_states_upload": [P(Problem), P(PlanInfo), P(Tensors), vp, vp, ctypes.c_size_t, P(Problem), P(PlanInfo),
                                vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp],
    "bsk_merge_state_pair": [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp],
    "bsk_run_noalloc": [P(Problem), P(PlanInfo), P(Tensors), vp, vp],
    "bsk_rope_table": [vp, i32, i32, f64, vp],
    "bsk_debug_gather": [P(Problem), P(PlanInfo), P(Tensors), vp, vp, vp, vp, vp],
    "bsk_debug_stream_read": [vp, ctypes.c_size_t, vp, ctypes.c_size_t, i32, vp],
    "bsk_debug_block_read": [vp, ctypes.c_size_t, vp, i32, vp, ctypes.c_size_t, i32, vp],
    "bsk_rope_apply": [P(Problem), i32, i32, vp, vp, vp, P(Tensors), vp, i64, i64, vp, vp],
    "bsk_append_paged_kv": [P(Problem), i32, i32, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, i64, i64, i64, i64, i64,
                            i64, vp],
}
for _name, _args in _sig.items():
    getattr(_lib, _name).restype = i32
    getattr(_lib, _name).argtypes = _args


class BskError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status
        self.message = message


def _ok(status: int):
    if status != OK:
        raise BskError(status, last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take a pointer of {type(x)}")


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def _nbytes(x) -> int:
    if isinstance(x, np.ndarray):
        return x.nbytes
    return x.numel() * x.element_size()


def status_string(status: int) -> str:
    return _lib.bsk_status_string(status).decode()


def last_error() -> str:
    return _lib.bsk_last_error().decode()


def device_workers(problem: Problem) -> int:
    out = i32(0)
    _ok(_lib.bsk_device_workers(ctypes.byref(problem), ctypes.byref(out)))
    return out.value


def workspace_query(problem: Problem):
    """-> (int_ws_bytes, float_ws_bytes, host_ws_bytes)"""
    a, b, c = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _ok(_lib.bsk_workspace_query(ctypes.byref(problem), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def plan(problem: Problem, qo_indptr, kv_len, kv_indptr, host_ws, int_ws=None, stream=None) -> PlanInfo:
    """Host arrays are int32 numpy arrays; host_ws a host buffer (numpy or pinned torch tensor);
    int_ws a device buffer or None (plan on the host only)."""
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kl = np.ascontiguousarray(kv_len, dtype=np.int32)
    ki = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    info = PlanInfo()
    _ok(_lib.bsk_plan(ctypes.byref(problem), int(len(kl)), qo.ctypes.data, kl.ctypes.data, ki.ctypes.data,
                      _ptr(host_ws), _nbytes(host_ws), _ptr(int_ws), 0 if int_ws is None else _nbytes(int_ws),
                      _stream(stream), ctypes.byref(info)))
    return info


def upload_plan(problem: Problem, info: PlanInfo, host_ws, int_ws, stream=None):
    """Copy a plan built on the host only (plan() without int_ws) into the int workspace."""
    _ok(_lib.bsk_upload_plan(ctypes.byref(problem), ctypes.byref(info), _ptr(host_ws), _nbytes(host_ws),
                             _ptr(int_ws), _nbytes(int_ws), _stream(stream)))


def run_decode(problem: Problem, info: PlanInfo, tensors: Tensors, int_ws, float_ws, stream=None):
    _ok(_lib.bsk_run_decode(ctypes.byref(problem), ctypes.byref(info), ctypes.byref(tensors), _ptr(int_ws),
                            _ptr(float_ws), 0 if float_ws is None else _nbytes(float_ws), _stream(stream)))


def run_prefill(problem: Problem, info: PlanInfo, tensors: Tensors, int_ws, float_ws, stream=None):
    _ok(_lib.bsk_run_prefill(ctypes.byref(problem), ctypes.byref(info), ctypes.byref(tensors), _ptr(int_ws),
                             _ptr(float_ws), 0 if float_ws is None else _nbytes(float_ws), _stream(stream)))


def merge_states(problem: Problem, info: PlanInfo, tensors: Tensors, int_ws, float_ws, stream=None):
    _ok(_lib.bsk_merge_states(ctypes.byref(problem), ctypes.byref(info), ctypes.byref(tensors), _ptr(int_ws),
                              _ptr(float_ws), 0 if float_ws is None else _nbytes(float_ws), _stream(stream)))


def merge_states_upload(problem: Problem, info: PlanInfo, tensors: Tensors, int_ws, float_ws, next_problem: Problem,
                        next_info: PlanInfo, next_host_ws, next_int_ws, stream=None):
    """merge_states of one run and upload_plan of the next plan (another int workspace), one launch."""
    _ok(_lib.bsk_merge_states_upload(ctypes.byref(problem), ctypes.byref(info), ctypes.byref(tensors), _ptr(int_ws),
                                     _ptr(float_ws), 0 if float_ws is None else _nbytes(float_ws),
                                     ctypes.byref(next_problem), ctypes.byref(next_info), _ptr(next_host_ws),
                                     _nbytes(next_host_ws), _ptr(next_int_ws), _nbytes(next_int_ws),
                                     _stream(stream)))


def run_noalloc(problem: Problem, info: PlanInfo, tensors: Tensors, int_ws, stream=None):
    _ok(_lib.bsk_run_noalloc(ctypes.byref(problem), ctypes.byref(info), ctypes.byref(tensors), _ptr(int_ws),
                             _stream(stream)))


def merge_state_pair(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows: int, head_dim: int, out_dtype: int,
                     stream=None):
    _ok(_lib.bsk_merge_state_pair(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out), _ptr(lse_out),
                                  rows, head_dim, out_dtype, _stream(stream)))


def rope_table(table, n_pos: int, head_dim: int, theta: float, stream=None):
    _ok(_lib.bsk_rope_table(_ptr(table), n_pos, head_dim, float(theta), _stream(stream)))


def append_paged_kv(problem: Problem, batch: int, n_total: int, append_indptr, kv_len, kv_page_indptr,
                    kv_page_indices, k_new, v_new, new_stride_tok: int, new_stride_head: int, k_cache, v_cache,
                    k_strides, v_strides, stream=None):
    """k_strides / v_strides: (page, head, token) element strides of the pools."""
    _ok(_lib.bsk_append_paged_kv(ctypes.byref(problem), batch, n_total, _ptr(append_indptr), _ptr(kv_len),
                                 _ptr(kv_page_indptr), _ptr(kv_page_indices), _ptr(k_new), _ptr(v_new),
                                 int(new_stride_tok), int(new_stride_head), _ptr(k_cache), _ptr(v_cache),
                                 *(int(x) for x in k_strides), *(int(x) for x in v_strides), _stream(stream)))


def rope_apply(problem: Problem, batch: int, max_kv_len: int, qo_indptr, kv_len, kv_page_indptr, tensors: Tensors,
               q_out, qo_stride_tok: int, qo_stride_head: int, k_out, stream=None):
    _ok(_lib.bsk_rope_apply(ctypes.byref(problem), batch, max_kv_len, _ptr(qo_indptr), _ptr(kv_len),
                            _ptr(kv_page_indptr), ctypes.byref(tensors), _ptr(q_out), int(qo_stride_tok),
                            int(qo_stride_head), _ptr(k_out), _stream(stream)))


def debug_gather(problem: Problem, info: PlanInfo, tensors: Tensors, int_ws, row_offsets, k_out, v_out,
                 stream=None):
    _ok(_lib.bsk_debug_gather(ctypes.byref(problem), ctypes.byref(info), ctypes.byref(tensors), _ptr(int_ws),
                              _ptr(row_offsets), _ptr(k_out), _ptr(v_out), _stream(stream)))


def debug_stream_read(src, sink, grid: int, stream=None):
    """Measurement hook: read all of src (a device buffer) once; sink receives one XOR word per
    thread."""
    _ok(_lib.bsk_debug_stream_read(_ptr(src), _nbytes(src), _ptr(sink), _nbytes(sink), int(grid), _stream(stream)))


def debug_block_read(src, order, sink, grid: int, stream=None):
    """Measurement hook: read the 4 KB blocks of src (a device buffer) listed in order (a device int32
    array of block indices); sink receives one XOR word per thread."""
    _ok(_lib.bsk_debug_block_read(_ptr(src), _nbytes(src), _ptr(order), int(order.numel()), _ptr(sink), _nbytes(sink),
                                  int(grid), _stream(stream)))


EXPORTED = ["bsk_status_string", "bsk_last_error", *_sig.keys()]
