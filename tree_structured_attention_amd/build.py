"""Build libtree_attn.so in-tree with hipcc for gfx950.

    python -m tree_structured_attention_amd.build

Host sources (plan builder, C ABI) and the HIP kernels are compiled to
objects under ``_build/`` and linked into
``tree_structured_attention_amd/libtree_attn.so``.  hipcc cross-compiles for
gfx950 without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtree_attn.so")

ARCH = os.environ.get("TREE_ATTN_ARCH", "gfx950")
HOST_SOURCES = ["plan.cpp", "api.cpp", "errors.cpp", "draft.cpp", "kv_pool.cpp"]
HIP_SOURCES = ["attn_kernels.hip", "bwd_kernels.hip", "accept_kernels.hip", "calib_kernels.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]
# Packed fp32 VALU ops are kept out of the device code on purpose.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the tree attention library needs ROCm's hipcc")


def _rocm_include() -> str:
    return os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "include")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{_rocm_include()}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
