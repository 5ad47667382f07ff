"""Builds libmoe.so (the gfx950 HIP kernels and the C ABI of include/moe.h) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
OBJDIR = os.path.join(ROOT, "_build", "moe")

HIP_SOURCES = ["router.hip", "permute.hip", "gemm.hip", "combine.hip", "norm.hip", "api.hip"]
CXX_SOURCES = ["plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    common = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC]
    jobs, objs = [], []
    for s in HIP_SOURCES:
        o = os.path.join(OBJDIR, s + ".o")
        # packed-fp32 instructions stay disabled in device code
        jobs.append([hipcc(), "--offload-arch=" + ARCH, "-c", *common, "-Xclang", "-target-feature",
                     "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
                     os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in CXX_SOURCES:
        o = os.path.join(OBJDIR, s + ".o")
        jobs.append(["g++", "-c", *common, "-Wall", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_compile, jobs))
    tmp = LIB + ".tmp%d" % os.getpid()
    _compile([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
