"""Build ``libduo.so`` in-tree: hipcc for the gfx950 kernels, g++ for the host-only C++.

Usage: ``python -m head_split_kv_amd.build`` (or ``__graft_entry__.build()``).
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libduo.so")
ARCH = "gfx950"

HIP_SOURCES = ["cache_kernels.hip", "decode.hip", "prefill.hip", "reorder.hip", "kv4.hip", "probe.hip"]
CXX_SOURCES = ["duo_host.cpp", "duo_api.cpp", "preprocess.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off (the compiler still emits plain fp32 FMAs)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source extra flags. decode.hip: the leading scalar kernel arguments arrive preloaded in
# SGPRs on gfx950 (up to 16 dwords): the decode kernels' work-item decomposition, so that a
# block's first argument loads do not wait on an earlier one, and every argument of the split
# merge kernel.
HIP_EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link ``head_split_kv_amd/libduo.so``; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *HIP_EXTRA.get(s, []), "-c", os.path.join(CSRC, s),
                     "-o", obj])
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([CXX, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj])
    with cf.ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
