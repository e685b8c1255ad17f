"""CPU oracle for the quantized prefill GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and the
two share no code: this side decodes the canonical codec bytes itself
(``qgemm_oracle.c``) in fp64 and contracts with a naive triple loop.

Functions follow the plain definitions stated in ``qgemm_oracle.c``:
exact fp64 decode of Q4_0 / MLX4-G64 / MLX4-G32 / Q2_0 / Q8_0 / Q4_K / ternary weights, ``ref = X * W^T`` with
``k`` ascending into one fp64 accumulator, ``SiLU(g) * u`` and ``GELU(g) * u`` (tanh form) in fp64.
Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library routines (numpy's correctly rounded float16 conversion, BLAS fp64
matmul), exact rational brute force and the codec facts printed on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qgemm_oracle.c")
LIB = os.path.join(HERE, "libqgemm_oracle.so")

Q4_0, MLX4_G64, Q2_0, Q8_0, MLX4_G32, Q4_K, TERNARY, TERNARY_Q2 = 1, 2, 3, 4, 5, 6, 7, 8

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, fp contraction off)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_f64_to_f16.argtypes = [ctypes.c_double]
        L.orc_f16_to_f64_array.argtypes = [p, p, i64]
        L.orc_f64_to_f16_array.argtypes = [p, p, i64]
        L.orc_block_geometry.argtypes = [i32, p, p]
        L.orc_block_geometry.restype = i32
        L.orc_decode_rows.argtypes = [i32, p, i64, i64, i64, i64, p]
        L.orc_decode_rows.restype = i32
        L.orc_dequant_f16_rows.argtypes = [i32, p, i64, i64, i64, i64, p, p]
        L.orc_dequant_f16_rows.restype = i32
        L.orc_matmul_xwt.argtypes = [p, i64, p, i64, i64, i64, p, i32]
        L.orc_swiglu.argtypes = [p, p, p, i64]
        L.orc_geglu.argtypes = [p, p, p, i64]
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().orc_f16_to_f64_array(_ptr(bits), _ptr(out), bits.size)
    return out


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f64_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def block_geometry(codec: int):
    w = ctypes.c_int64()
    b = ctypes.c_int64()
    ok = lib().orc_block_geometry(codec, ctypes.byref(w), ctypes.byref(b))
    if not ok:
        raise ValueError(f"unknown codec {codec}")
    return w.value, b.value


def decode(codec: int, canon: np.ndarray, n: int, k: int, row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """Exact fp64 decode of rows [row0, row0+nrows) of an [n, k] weight matrix."""
    if nrows is None:
        nrows = n - row0
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    out = np.empty((nrows, k), dtype=np.float64)
    rc = lib().orc_decode_rows(codec, _ptr(canon), n, k, row0, nrows, _ptr(out))
    if rc == -2:
        raise ValueError("oracle decode found an invalid code byte")
    if rc:
        raise ValueError("oracle decode rejected codec/shape")
    return out


def dequant_f16_bits(codec: int, canon: np.ndarray, n: int, k: int, row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """Each exact weight rounded once to binary16; returns uint16 bit patterns."""
    if nrows is None:
        nrows = n - row0
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    scratch = np.empty((nrows, k), dtype=np.float64)
    out = np.empty((nrows, k), dtype=np.uint16)
    rc = lib().orc_dequant_f16_rows(codec, _ptr(canon), n, k, row0, nrows, _ptr(scratch), _ptr(out))
    if rc:
        raise ValueError("oracle dequant rejected codec/shape")
    return out


def matmul_xwt(x: np.ndarray, w: np.ndarray, threads: int = 0) -> np.ndarray:
    """ref = X * W^T with X fp16 [m, k] (any float16 array) and W fp64 [n, k]."""
    xb = np.ascontiguousarray(x).view(np.uint16) if x.dtype == np.float16 else np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float64)
    m, k = xb.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("K mismatch")
    out = np.empty((m, n), dtype=np.float64)
    lib().orc_matmul_xwt(_ptr(xb), k, _ptr(w), m, n, k, _ptr(out), threads)
    return out


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.empty(g.shape, dtype=np.float64)
    lib().orc_swiglu(_ptr(g), _ptr(u), _ptr(out), g.size)
    return out


def geglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.empty(g.shape, dtype=np.float64)
    lib().orc_geglu(_ptr(g), _ptr(u), _ptr(out), g.size)
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


def canonical_rows(codec: int, canon: np.ndarray, n: int, k: int, rows: np.ndarray) -> np.ndarray:
    """Canonical bytes of a row subset (byte selection only, no arithmetic)."""
    rows = np.asarray(rows, dtype=np.int64)
    if codec == Q4_0:
        return np.ascontiguousarray(canon.reshape(n, -1)[rows]).reshape(-1)
    if codec in (Q2_0, Q8_0, Q4_K, TERNARY, TERNARY_Q2):
        return np.ascontiguousarray(canon.reshape(n, -1)[rows]).reshape(-1)
    group = 32 if codec == MLX4_G32 else 64
    codes = canon[: n * k // 2].reshape(n, -1)[rows]
    sc = canon[n * k // 2: n * k // 2 + n * (k // group) * 2].reshape(n, -1)[rows]
    bi = canon[n * k // 2 + n * (k // group) * 2:].reshape(n, -1)[rows]
    return np.concatenate([codes.reshape(-1), sc.reshape(-1), bi.reshape(-1)])


def gemm_ref(codec: int, canon: np.ndarray, n: int, k: int, x: np.ndarray,
             rows_n=None, threads: int = 0) -> np.ndarray:
    """ref[m, j] = sum_k x[m,k] * w[rows_n[j], k] (all rows when rows_n is None)."""
    if rows_n is None:
        w = decode(codec, canon, n, k)
    else:
        sub = canonical_rows(codec, canon, n, k, rows_n)
        w = decode(codec, sub, len(rows_n), k)
    return matmul_xwt(x, w, threads)


def swiglu_ref(codec: int, canon_g: np.ndarray, canon_u: np.ndarray, n: int, k: int,
               x: np.ndarray, rows_n=None, threads: int = 0) -> np.ndarray:
    g = gemm_ref(codec, canon_g, n, k, x, rows_n, threads)
    u = gemm_ref(codec, canon_u, n, k, x, rows_n, threads)
    return swiglu(g, u)


def geglu_ref(codec: int, canon_g: np.ndarray, canon_u: np.ndarray, n: int, k: int,
              x: np.ndarray, rows_n=None, threads: int = 0) -> np.ndarray:
    g = gemm_ref(codec, canon_g, n, k, x, rows_n, threads)
    u = gemm_ref(codec, canon_u, n, k, x, rows_n, threads)
    return geglu(g, u)
