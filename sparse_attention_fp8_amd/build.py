"""Build libdsa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python sparse_attention_fp8_amd/build.py      # or __graft_entry__.build()

(Run it as a script: importing the package loads the library it builds.)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
ARCH = "gfx950"

SOURCES = ["indexer.hip", "topk.hip", "attention.hip", "project.hip", "train.hip", "mha.hip",
           "noalloc.hip", "dsa_api.cpp"]
# per-source code generation options
EXTRA = {
    # keep MFMA results in VGPRs: the indexer epilogue reads every result with VALU
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "train.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # a register array indexed at run time must show up as scratch, not be
            # moved to LDS behind the kernels' backs (that also reads the work-group
            # size from the dispatch packet in host memory)
            "-mllvm", "-disable-promote-alloca-to-lds",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def _compile(src: str, hipcc: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libdsa.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
