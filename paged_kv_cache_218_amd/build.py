"""Build libpagedattn.so in-tree for gfx950 (hipcc) from csrc/.

    python -m paged_kv_cache_218_amd.build [-v]

The host bookkeeping (pool.cpp) is plain C++ compiled by g++; the HIP sources
are compiled by hipcc for gfx950 only, with packed-FP32 instruction selection
turned off; everything links into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["attention.hip", "kvwrite.hip", "spec.hip", "probe.hip"]
HOST_SOURCES = ["pool.cpp", "prefix_cache.cpp"]
HIP_FLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra"]


def _run(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for cmd, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature name; that warning is noise
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
        if verbose and lines:
            print("\n".join(lines))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    _run(cmds, verbose)
    tmp = LIB + ".tmp"
    _run([[HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
