"""Build libqgemm.so (HIP kernels for gfx950 + the C-ABI) in-tree with hipcc.

Run ``python -m quantized_prefill_gemm_codec_amd.build``.  hipcc cross-compiles
the device code, so this works on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libqgemm.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIP_SOURCES = ["gemm.hip", "gemv.hip", "attention.hip", "api.hip"]
CXX_SOURCES = ["pack.cpp"]
HEADERS = ["planar.h", "unpack.h", "launch.h", "lds_dma.h"]

# -packed-fp32-ops is switched off for all device code: the compiler then never
# forms v_pk_{add,mul,fma}_f32 from scalar fp32 code.
HIPCC_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libqgemm.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libqgemm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES + CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        flags = HIPCC_FLAGS if src.endswith(".hip") else ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
        compiler = cc if src.endswith(".hip") else "g++"
        jobs.append([compiler, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for r in ex.map(_run, jobs):
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
