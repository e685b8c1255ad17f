"""Build libqgemm.so (HIP kernels for gfx950 + the C-ABI) in-tree with hipcc.

Run ``python -m quantized_prefill_gemm_codec_amd.build``.  hipcc cross-compiles
the device code, so this works on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libqgemm.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIP_SOURCES = ["gemm.hip", "gemv.hip", "attention.hip", "api.hip"]
CXX_SOURCES = ["pack.cpp"]
HEADERS = ["planar.h", "unpack.h", "launch.h", "lds_dma.h", "dispatch.h", "kutil.h"]

# -packed-fp32-ops is switched off for all device code: the compiler then never
# forms v_pk_{add,mul,fma}_f32 from scalar fp32 code.
# -Werror: the sources compile without a single warning.  The resource-usage
# remarks give every kernel's registers, scratch and LDS, checked below.
HIPCC_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Rpass-analysis=kernel-resource-usage",
               f"-I{os.path.join(ROOT, 'include')}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror"]
RESOURCES = os.path.join(BUILD, "kernel_resources.txt")
ROUNDING = os.path.join(BUILD, "q4_k_rounding.txt")
LDS_MAX = 160 * 1024   # bytes of LDS per compute unit on gfx950

# Kernels that unpack Q4_K weights to fp16 (codec 6): the GEMM tiles and the
# dequant kernel.  The GEMV dots raw codes and rounds no weight.
Q4_K_UNPACK = re.compile(r"(gemm_dma_kernel|gemm_kernel|dequant_kernel)ILi6E")


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


def _demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
        out = r.stdout.splitlines()
        return out if len(out) == len(names) else list(names)
    except (OSError, subprocess.CalledProcessError):
        return list(names)


def kernel_resources(stderr: str):
    """Per-kernel resource remarks of one hipcc run: {name: {field: value}}."""
    kernels, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return kernels


def check_resources(kernels):
    """Every kernel runs without scratch memory (no register spills, no
    dynamic stack) and within the LDS of one compute unit; returns the table
    lines, raises RuntimeError listing every kernel that breaks a budget."""
    names = sorted(kernels)
    pretty = _demangle(names)
    lines, bad = [], []
    for raw, name in zip(names, pretty):
        r = kernels[raw]
        scratch = int(r.get("ScratchSize [bytes/lane]", "0"))
        spills = int(r.get("VGPRs Spill", "0")) + int(r.get("SGPRs Spill", "0"))
        lds = int(r.get("LDS Size [bytes/block]", "0"))
        dyn = r.get("Dynamic Stack", "False") != "False"
        lines.append(f"{name}: VGPRs={r.get('VGPRs')} AGPRs={r.get('AGPRs')} SGPRs={r.get('TotalSGPRs')} "
                     f"scratch={scratch} spills={spills} LDS={lds} occupancy={r.get('Occupancy [waves/SIMD]')}")
        if scratch or spills or dyn or lds > LDS_MAX:
            bad.append(lines[-1])
    if bad:
        raise RuntimeError("kernels over their resource budget (scratch, spills, dynamic stack or LDS):\n" +
                           "\n".join(bad))
    return lines


def llvm_tool(name: str) -> str:
    """An LLVM tool of the ROCm toolchain that hipcc drives."""
    roots = [os.environ.get("ROCM_PATH"), os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "/opt/rocm"]
    for root in roots:
        if root:
            cand = os.path.join(root, "lib", "llvm", "bin", name)
            if os.path.exists(cand):
                return cand
    raise RuntimeError(f"{name} not found beside hipcc")


def device_mnemonics(obj: str) -> dict:
    """{kernel symbol: {mnemonic: count}} of the gfx950 code object inside a
    host object built here (its offload bundle, disassembled)."""
    with tempfile.TemporaryDirectory() as tmp:
        fat, co = os.path.join(tmp, "fat.bin"), os.path.join(tmp, "dev.co")
        _run([llvm_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, os.path.join(tmp, "host.o")])
        _run([llvm_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
              f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"])
        text = _run([llvm_tool("llvm-objdump"), "-d", f"--mcpu={ARCH}", co]).stdout
    return parse_disassembly(text)


def parse_disassembly(text: str) -> dict:
    funcs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            cur = funcs.setdefault(m.group(1), {})
            continue
        if cur is not None and line[:1].isspace():
            tok = line.split()
            if tok and re.match(r"^[sv]_[a-z0-9_]+$", tok[0]):
                cur[tok[0]] = cur.get(tok[0], 0) + 1
    return funcs


def check_single_rounding(funcs: dict):
    """Q4_K weights are the correctly rounded fp16 value of d sc q - dmin m.
    The unpack writes the fused multiply-add narrowed to fp16 in plain C and
    relies on hipcc selecting v_fma_mixlo_f16 / v_fma_mixhi_f16, which round
    the exact result once; a lowering through v_fma_mix_f32 and a separate
    conversion would round twice.  Every Q4_K unpacking kernel must use the
    former and not the latter; returns the table lines, raises RuntimeError
    naming every kernel that breaks this (or if none is found)."""
    names = sorted(n for n in funcs if Q4_K_UNPACK.search(n))
    lines, bad = [], []
    for raw, name in zip(names, _demangle(names)):
        f = funcs[raw]
        lo, hi = f.get("v_fma_mixlo_f16", 0), f.get("v_fma_mixhi_f16", 0)
        wide = f.get("v_fma_mix_f32", 0) + f.get("v_mad_mix_f32", 0)
        lines.append(f"{name}: v_fma_mixlo_f16={lo} v_fma_mixhi_f16={hi} v_fma_mix_f32={wide}")
        if lo == 0 or hi == 0 or wide:
            bad.append(lines[-1])
    if not names:
        raise RuntimeError("no Q4_K unpacking kernel found in the device code")
    if bad:
        raise RuntimeError("Q4_K kernels whose unpack may round twice:\n" + "\n".join(bad))
    return lines


def build(verbose: bool = False) -> str:
    """Compile every source and link libqgemm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES + CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        flags = HIPCC_FLAGS if src.endswith(".hip") else CXX_FLAGS
        compiler = cc if src.endswith(".hip") else "g++"
        jobs.append([compiler, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    kernels = {}
    with cf.ThreadPoolExecutor(workers) as ex:
        for r in ex.map(_run, jobs):
            kernels.update(kernel_resources(r.stderr))
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    table = check_resources(kernels)
    with open(RESOURCES, "w") as f:
        f.write("\n".join(table) + "\n")
    funcs = {}
    for src in ("gemm.hip", "gemv.hip"):
        funcs.update(device_mnemonics(os.path.join(BUILD, src + ".o")))
    rounding = check_single_rounding(funcs)
    with open(ROUNDING, "w") as f:
        f.write("\n".join(rounding) + "\n")
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
