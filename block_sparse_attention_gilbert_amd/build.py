"""Build libbsa.so (HIP, gfx950) in-tree.

    python block_sparse_attention_gilbert_amd/build.py

Every call recompiles all sources: object files go to ``_build/`` at the
repository root and the shared library to this package's directory.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsa.so")

ARCH = "gfx950"
HIP_SOURCES = ["gilbert.hip", "route.hip", "attn.hip", "geometry.hip", "diag.hip", "api.hip"]
HOST_SOURCES = ["validate.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC]
# Packed fp32 VALU instructions stay disabled in device code.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), r.stdout))
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libbsa.so``; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([hipcc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        jobs.append([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[j.index("-o") + 1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
