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
    assert len(names) == 13, names
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
  F(bsk_problem, rope_theta) F(bsk_problem, sm_scale) F(bsk_problem, max_merge)
  F(bsk_plan_info, total_cost) F(bsk_plan_info, used_bytes)
  F(bsk_tensors, kv_page_indices) F(bsk_tensors, lse_stride_tok) F(bsk_tensors, rope_n_pos)
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
