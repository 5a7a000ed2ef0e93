"""Builds libqdm.so in-tree: host C++ with g++, gfx950 kernels with hipcc.

    python quantized_decode_mlp_amd/build.py      (run by path: importing the
                                                  package would load the old library)

The host quantizer/packer is compiled with -ffp-contract=off and no
fast-math (its fp64 steps must stay single IEEE operations).  Kernels are
compiled for gfx950 only, with packed-fp32 instruction selection disabled.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqdm.so")

ARCH = "gfx950"
HOST_SOURCES = ["qdm_pack.cpp", "qdm_api.cpp"]
HIP_SOURCES = ["qdm_gemv.hip", "qdm_mfma.hip", "qdm_mma_stream.hip", "qdm_mma_down.hip", "qdm_rmsnorm.hip",
               "qdm_chain.hip", "qdm_prefill.hip", "qdm_noalloc.hip"]

HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-pthread",
              "-Wall", "-Wextra", "-Wno-unused-parameter"]
HIP_FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-parameter"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return p


def build(verbose: bool = False) -> str:
    """Compiles every source and links libqdm.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, "-pthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
