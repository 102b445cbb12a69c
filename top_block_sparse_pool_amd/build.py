"""Build the HIP library in-tree: hipcc for gfx950, one object per source, then link.

Usage: python -m top_block_sparse_pool_amd.build   (or call build()).
The result is top_block_sparse_pool_amd/libattn_tbs.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libattn_tbs.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["csrc/abi.cpp", "csrc/router.hip", "csrc/schedule.hip", "csrc/augment.hip", "csrc/quant.hip",
           "csrc/flash_fwd.hip", "csrc/noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    # Packed fp32 VALU ops are kept out of all generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the online softmax rescales them with VALU
    # ops, and AGPR accumulators would be copied back and forth every tile.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *COMMON, *lang, "-c", os.path.join(PKG, src), "-o", obj])
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
