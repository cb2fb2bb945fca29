"""Build libbsk.so in-tree with hipcc for gfx950.

    python block_sparse_kv_plan_amd/build.py      (or __graft_entry__.build())

(run as a script, not ``-m``: importing the package would load the library being rebuilt)

Every translation unit is compiled in parallel into ``_build/`` and linked
into ``block_sparse_kv_plan_amd/libbsk.so``.  The planner (plan.cpp) is
plain C++17 and also builds with g++ alone for host-side sanitizer runs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsk.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed-fp32 instructions are kept out of the device code on purpose
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]
DEVICE_SOURCES = ["decode.hip", "prefill.hip", "mixed.hip", "merge.hip", "append.hip", "rope.hip", "noalloc.hip"]
# per-file extras: the prefill kernel's logits are never NaN when they reach fmaxf (masked ones are
# -inf), so it is built without NaN semantics and its max needs no operand canonicalisation
EXTRA = {"prefill.hip": ["-fno-honor-nans"], "mixed.hip": ["-fno-honor-nans"]}
HOST_SOURCES = ["plan.cpp", "capi.cpp"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, f"--offload-arch={ARCH}", *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, f"--offload-arch={ARCH}", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [os.path.join(BUILD, s + ".o") for s in DEVICE_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
