"""Builds libsplitk.so (the HIP library) in-tree for gfx950 with hipcc.

Usage: ``python -m split_dense_gemm_amd.build`` (also called by
``__graft_entry__.build()``).  Every call compiles from source.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsplitk.so")
SOURCES = ["gemm_bt.hip", "plan.cpp", "slab_reduce.hip", "split_choice.cpp", "splitk_api.cpp", "static_slabs.hip"]
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from forming packed F32 VALU ops.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj_dir: str, extra) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]  # the .cpp file includes HIP launch APIs as well
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    return obj


def build(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, list(extra_flags)), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
