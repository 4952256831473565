"""Build libqlinear.so (HIP kernels for gfx950 + host quantisers) in-tree.

    python -m weight_quantized_amd.build        # or build() from Python

HIP sources are compiled with hipcc for gfx950 only; host C++ sources with
ROCm's clang++.  Packed-fp32 instructions are disabled in device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqlinear.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["w4a16.hip", "w8a8.hip", "kv_int8.hip"]
HOST_SOURCES = ["status.cpp", "host_quant.cpp"]

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-mf16c", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
              "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC, f"-I{ROCM}/include"]


def _hipcc():
    return shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")


def _clangxx():
    cand = os.path.join(ROCM, "llvm", "bin", "clang++")
    return cand if os.path.exists(cand) else (shutil.which("clang++") or "g++")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libqlinear.so next to this file."""
    tmpdir = tempfile.mkdtemp(prefix="qlbuild_")
    try:
        jobs = []
        objs = []
        for s in HIP_SOURCES:
            o = os.path.join(tmpdir, s + ".o")
            jobs.append([_hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
            objs.append(o)
        for s in HOST_SOURCES:
            o = os.path.join(tmpdir, s + ".o")
            jobs.append([_clangxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
            objs.append(o)
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        _run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib, *objs, "-lpthread"], verbose)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
