"""Python binding of libqgemm.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C-ABI in
``include/qgemm.h``; this module checks tensor dtypes, devices and strides,
flattens leading batch dimensions (the pages' quantized linear layer accepts
arbitrary leading dims: releases page, v0.3.0), allocates outputs with torch
and passes raw pointers plus torch's current HIP stream.  There is no CPU
fallback: if the library is not built, every entry point raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

QG_CODEC_Q4_0 = 1
QG_CODEC_MLX4_G64 = 2
QG_CODEC_Q2_0 = 3
QG_CODEC_Q8_0 = 4
QG_CODEC_MLX4_G32 = 5
QG_CODEC_Q4_K = 6
QG_CODEC_TERNARY_1_58 = 7
QG_CODEC_TERNARY_1_58_Q2 = 8
CODECS = {"q4_0": QG_CODEC_Q4_0, "mlx4_g64": QG_CODEC_MLX4_G64, "q2_0": QG_CODEC_Q2_0, "q8_0": QG_CODEC_Q8_0,
          "mlx4_g32": QG_CODEC_MLX4_G32, "q4_k": QG_CODEC_Q4_K, "ternary": QG_CODEC_TERNARY_1_58,
          "ternary_q2": QG_CODEC_TERNARY_1_58_Q2}
BLOCK = {QG_CODEC_Q4_0: 32, QG_CODEC_MLX4_G64: 64, QG_CODEC_Q2_0: 128, QG_CODEC_Q8_0: 32, QG_CODEC_MLX4_G32: 32,
         QG_CODEC_Q4_K: 256, QG_CODEC_TERNARY_1_58: 256, QG_CODEC_TERNARY_1_58_Q2: 256}

QG_OK = 0
STATUS = {0: "QG_OK", -1: "QG_ERR_NULL", -2: "QG_ERR_CODEC", -3: "QG_ERR_SHAPE", -4: "QG_ERR_ALIGN",
          -5: "QG_ERR_MISMATCH", -6: "QG_ERR_LAUNCH", -7: "QG_ERR_SIZE",
          -8: "QG_ERR_CODE"}

EXPORTS = ("qgemm_prefill", "qgemm_prefill_heads", "qgemm_swiglu", "qgemm_geglu", "qgemv_decode", "qg_packed_sizes",
           "qg_canonical_size", "qg_pack_host", "qg_dequant", "qg_kernel_for", "qg_stream_read", "qg_status_str",
           "qg_version", "qattn_prefill_q8kv", "qg_pack_kv_host")

# entry ids of qg_kernel_for
ENTRY = {"prefill": 0, "heads": 1, "swiglu": 2, "geglu": 3, "gemv": 4}


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_str(status)})")


class qg_weight(ctypes.Structure):
    _fields_ = [("codec", ctypes.c_int32), ("flags", ctypes.c_int32), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("qs", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libqgemm.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_prefill_gemm_codec_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, p, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        W = ctypes.POINTER(qg_weight)
        L.qgemm_prefill.argtypes = [W, p, i64, i64, p, i64, p]
        L.qgemm_swiglu.argtypes = [W, W, p, i64, i64, p, i64, p]
        L.qgemm_prefill_heads.argtypes = [W, p, i64, i64, p, i64, p]
        L.qgemm_geglu.argtypes = [W, W, p, i64, i64, p, i64, p]
        L.qgemv_decode.argtypes = [W, p, i64, i64, p, i64, p]
        L.qg_packed_sizes.argtypes = [i32, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.qg_canonical_size.argtypes = [i32, i64, i64, ctypes.POINTER(sz)]
        L.qg_pack_host.argtypes = [i32, i64, i64, p, sz, p, p]
        L.qg_dequant.argtypes = [W, p, i64, p]
        L.qg_stream_read.argtypes = [p, sz, p, p]
        L.qg_kernel_for.argtypes = [i32, i32, i64, i64, i64, ctypes.c_char_p, sz]
        L.qattn_prefill_q8kv.argtypes = [p, p, i64, i64, i64, p, p, p, p, i64, i64, i32, ctypes.c_float, p]
        L.qg_pack_kv_host.argtypes = [p, sz, i64, i64, p, p]
        L.qg_status_str.argtypes = [ctypes.c_int]
        L.qg_status_str.restype = ctypes.c_char_p
        L.qg_version.restype = i32
        for f in ("qgemm_prefill", "qgemm_prefill_heads", "qgemm_swiglu", "qgemm_geglu", "qgemv_decode", "qg_packed_sizes", "qg_canonical_size",
                  "qg_pack_host", "qg_dequant", "qg_kernel_for", "qg_stream_read", "qattn_prefill_q8kv",
                  "qg_pack_kv_host"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_str(st: int) -> str:
    try:
        return lib().qg_status_str(st).decode()
    except Exception:  # library unavailable while formatting an error
        return "?"


def _check(st: int, where: str):
    if st != QG_OK:
        raise QGError(st, where)


# ----------------------------------------------------------------- host side --

def qg_packed_sizes(codec: int, n: int, k: int):
    qs, sc = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().qg_packed_sizes(codec, n, k, ctypes.byref(qs), ctypes.byref(sc)), "qg_packed_sizes")
    return qs.value, sc.value


def qg_canonical_size(codec: int, n: int, k: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().qg_canonical_size(codec, n, k, ctypes.byref(b)), "qg_canonical_size")
    return b.value


def qg_pack_host(codec: int, n: int, k: int, canonical: np.ndarray):
    """Canonical codec bytes -> (qs, scales) planar planes as numpy uint8 arrays."""
    canonical = np.ascontiguousarray(canonical, dtype=np.uint8)
    qs_b, sc_b = qg_packed_sizes(codec, n, k)
    qs = np.empty(qs_b, dtype=np.uint8)
    sc = np.empty(sc_b, dtype=np.uint8)
    _check(lib().qg_pack_host(codec, n, k, canonical.ctypes.data, canonical.size, qs.ctypes.data, sc.ctypes.data),
           "qg_pack_host")
    return qs, sc


def qg_kernel_for(entry, codec: int, m: int, n: int, k: int) -> str:
    """Name of the kernel instantiation the entry point ('prefill', 'heads',
    'swiglu', 'geglu', 'gemv' or its id) would launch for these sizes."""
    e = ENTRY[entry] if isinstance(entry, str) else int(entry)
    buf = ctypes.create_string_buffer(128)
    _check(lib().qg_kernel_for(e, codec, m, n, k, buf, len(buf)), "qg_kernel_for")
    return buf.value.decode()


# --------------------------------------------------------------- device side --

def _torch():
    import torch
    return torch


class QWeight:
    """A packed weight matrix resident in device memory (torch-owned planes)."""

    def __init__(self, codec: int, n: int, k: int, qs, scales):
        self.codec, self.n, self.k = int(codec), int(n), int(k)
        self.qs, self.scales = qs, scales
        self._desc = qg_weight(self.codec, 0, self.n, self.k, qs.data_ptr(), scales.data_ptr())

    @classmethod
    def from_canonical(cls, codec: int, n: int, k: int, canonical: np.ndarray, device="cuda"):
        torch = _torch()
        qs, sc = qg_pack_host(codec, n, k, canonical)
        return cls(codec, n, k, torch.from_numpy(qs).to(device), torch.from_numpy(sc).to(device))

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def nbytes(self) -> int:
        return self.qs.numel() + self.scales.numel()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _as_rows(x, k: int):
    """Flatten leading dims to [M, K] rows with a 16-byte aligned row stride."""
    torch = _torch()
    if x.dtype != torch.float16 or not x.is_cuda:
        raise TypeError("x must be a float16 tensor on a HIP device")
    if x.dim() < 1 or x.shape[-1] != k:
        raise ValueError(f"x has K={x.shape[-1] if x.dim() else None}, weights expect K={k}")
    lead = tuple(x.shape[:-1])
    x2 = x.reshape(-1, k)
    m = x2.shape[0]
    if x2.stride(-1) != 1 or (m > 1 and x2.stride(0) % 8) or x2.data_ptr() % 16:
        x2 = x2.contiguous()
    ldx = x2.stride(0) if m > 1 else k
    return x2, lead, ldx


def _check_weights(device, *ws):
    for w in ws:
        if w.qs.device != device or w.scales.device != device:
            raise ValueError(f"weight planes are on {w.qs.device}, activations on {device}")


def _check_out_device(out, device):
    torch = _torch()
    if out.dtype != torch.float16 or not out.is_cuda or out.device != torch.device(device):
        raise ValueError(f"out must be a float16 tensor on {device} (got {out.dtype} on {out.device})")


def _out(m: int, n: int, device, out=None):
    """Output rows [M, N] with a row stride that is a multiple of 8 elements.
    A caller's `out` must be viewable as [M, N] rows of unit column stride on
    the device of X: the kernel writes straight into it, never into a copy."""
    torch = _torch()
    if out is not None:
        _check_out_device(out, device)
        try:
            o2 = out.view(-1, n)
        except RuntimeError as e:
            raise ValueError("out cannot be viewed as [M, N] rows without a copy") from e
        if o2.stride(-1) != 1 or o2.shape[0] != m:
            raise ValueError("out must be float16 [..., N] with M rows and unit column stride")
        return o2, (o2.stride(0) if m > 1 else 8 * ((n + 7) // 8)), out
    ldy = 8 * ((n + 7) // 8)
    buf = torch.empty((m, ldy), dtype=torch.float16, device=device)
    return buf, ldy, buf[:, :n]


def _no_rows(lead, n: int, device, out):
    """The result of a call with no rows of X (the C-ABI takes M >= 1): an
    empty [..., N] tensor, or the caller's `out` once it is checked."""
    torch = _torch()
    if out is None:
        return torch.empty((*lead, n), dtype=torch.float16, device=device)
    _check_out_device(out, device)
    if out.numel() != 0 or out.dim() < 1 or out.shape[-1] != n:
        raise ValueError("out must be float16 [..., N] with no rows")
    return out


def qgemm_prefill(w: QWeight, x, out=None, stream=None):
    """Y = X W^T for fp16 X [..., K]; returns fp16 [..., N]."""
    x2, lead, ldx = _as_rows(x, w.k)
    _check_weights(x.device, w)
    m = x2.shape[0]
    if m == 0:
        return _no_rows(lead, w.n, x.device, out)
    ybuf, ldy, y = _out(m, w.n, x.device, out)
    _check(lib().qgemm_prefill(w.desc, x2.data_ptr(), m, ldx, ybuf.data_ptr(), ldy, _stream(stream)),
           "qgemm_prefill")
    return y.reshape(*lead, w.n) if out is None else out


def qgemm_swiglu(wg: QWeight, wu: QWeight, x, out=None, stream=None):
    """SiLU(X Wg^T) * (X Wu^T) for fp16 X [..., K]; returns fp16 [..., N]."""
    x2, lead, ldx = _as_rows(x, wg.k)
    _check_weights(x.device, wg, wu)
    m = x2.shape[0]
    if m == 0:
        return _no_rows(lead, wg.n, x.device, out)
    ybuf, ldy, y = _out(m, wg.n, x.device, out)
    _check(lib().qgemm_swiglu(wg.desc, wu.desc, x2.data_ptr(), m, ldx, ybuf.data_ptr(), ldy, _stream(stream)),
           "qgemm_swiglu")
    return y.reshape(*lead, wg.n) if out is None else out


def qgemm_prefill_heads(w: QWeight, x, head_dim: int, out=None, stream=None):
    """Y = X W^T for fp16 X [M, K] written head-major: returns fp16 [N / head_dim, M, head_dim]."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("qgemm_prefill_heads takes a 2-D X [M, K]")
    x2, _, ldx = _as_rows(x, w.k)
    _check_weights(x.device, w)
    m = x2.shape[0]
    if m == 0:
        if head_dim < 8 or head_dim % 8 or w.n % head_dim:
            raise ValueError("head_dim must be a multiple of 8 that divides N")
        if out is None:
            return torch.empty((w.n // head_dim, 0, head_dim), dtype=torch.float16, device=x.device)
        _check_out_device(out, x.device)
        if out.numel() != 0:
            raise ValueError("out must be empty when X has no rows")
        return out
    if out is None:
        out = torch.empty((w.n // head_dim if head_dim else 0, m, head_dim), dtype=torch.float16, device=x.device)
    _check_out_device(out, x.device)
    if not out.is_contiguous() or out.numel() != m * w.n:
        raise ValueError("out must be a contiguous fp16 tensor of M * N elements")
    _check(lib().qgemm_prefill_heads(w.desc, x2.data_ptr(), m, ldx, out.data_ptr(), head_dim, _stream(stream)),
           "qgemm_prefill_heads")
    return out


def qgemm_geglu(wg: QWeight, wu: QWeight, x, out=None, stream=None):
    """GELU(X Wg^T) * (X Wu^T) (tanh-form GELU) for fp16 X [..., K]; returns fp16 [..., N]."""
    x2, lead, ldx = _as_rows(x, wg.k)
    _check_weights(x.device, wg, wu)
    m = x2.shape[0]
    if m == 0:
        return _no_rows(lead, wg.n, x.device, out)
    ybuf, ldy, y = _out(m, wg.n, x.device, out)
    _check(lib().qgemm_geglu(wg.desc, wu.desc, x2.data_ptr(), m, ldx, ybuf.data_ptr(), ldy, _stream(stream)),
           "qgemm_geglu")
    return y.reshape(*lead, wg.n) if out is None else out


def qgemv_decode(w: QWeight, x, out=None, stream=None):
    """Weight-streaming Y = X W^T for 1 <= M <= 64 rows of X."""
    x2, lead, ldx = _as_rows(x, w.k)
    _check_weights(x.device, w)
    m = x2.shape[0]
    if m == 0:
        return _no_rows(lead, w.n, x.device, out)
    ybuf, ldy, y = _out(m, w.n, x.device, out)
    _check(lib().qgemv_decode(w.desc, x2.data_ptr(), m, ldx, ybuf.data_ptr(), ldy, _stream(stream)),
           "qgemv_decode")
    return y.reshape(*lead, w.n) if out is None else out


def qg_dequant(w: QWeight, stream=None):
    """fp16 image [N, K] of the weights, from the kernels' unpack routines."""
    torch = _torch()
    ldw = 8 * ((w.k + 7) // 8)
    buf = torch.empty((w.n, ldw), dtype=torch.float16, device=w.qs.device)
    _check(lib().qg_dequant(w.desc, buf.data_ptr(), ldw, _stream(stream)), "qg_dequant")
    return buf[:, :w.k]


QG_STREAM_READ_SLOTS = 4096


def qg_stream_read(src, out=None, stream=None):
    """XOR of the 32-bit words of the contiguous device tensor src (its byte
    size a multiple of 16), read once by the streaming-read calibration kernel.
    With `out` (a device int32 tensor of QG_STREAM_READ_SLOTS elements) the
    per-wave partial XORs accumulate into it on the stream and nothing is
    synchronized; otherwise the XOR over fresh slots is returned."""
    torch = _torch()
    if not src.is_contiguous():
        raise ValueError("qg_stream_read needs a contiguous tensor")
    slots = out if out is not None else torch.zeros(QG_STREAM_READ_SLOTS, dtype=torch.int32, device=src.device)
    if slots.numel() < QG_STREAM_READ_SLOTS or slots.dtype != torch.int32:
        raise ValueError(f"qg_stream_read needs an int32 tensor of {QG_STREAM_READ_SLOTS} slots")
    nbytes = src.numel() * src.element_size()
    _check(lib().qg_stream_read(src.data_ptr(), nbytes, slots.data_ptr(), _stream(stream)), "qg_stream_read")
    if out is not None:
        return None
    return int(np.bitwise_xor.reduce(slots.cpu().numpy().view(np.uint32)))


class Q8KVCache:
    """Planar Q8_0 KV cache on the device: int8 codes [rows, D] and fp16 scales
    [rows, D / 32] for K and for V (rows = kv_heads * s)."""

    def __init__(self, kv_heads: int, s: int, head_dim: int, k_codes, k_scales, v_codes, v_scales):
        self.kv_heads, self.s, self.head_dim = kv_heads, s, head_dim
        self.k_codes, self.k_scales, self.v_codes, self.v_scales = k_codes, k_scales, v_codes, v_scales

    @classmethod
    def from_canonical(cls, kv_heads: int, s: int, head_dim: int, k_canonical: np.ndarray,
                       v_canonical: np.ndarray, device="cuda"):
        """Split canonical Q8_0 rows (qg_pack_kv_host) and upload."""
        torch = _torch()
        parts = []
        for canon in (k_canonical, v_canonical):
            canon = np.ascontiguousarray(canon, dtype=np.uint8)
            rows = kv_heads * s
            codes = np.empty(rows * head_dim, np.uint8)
            scales = np.empty(rows * (head_dim // 32) * 2, np.uint8)
            _check(lib().qg_pack_kv_host(canon.ctypes.data, canon.size, rows, head_dim, codes.ctypes.data,
                                         scales.ctypes.data), "qg_pack_kv_host")
            parts += [torch.from_numpy(codes).to(device), torch.from_numpy(scales).to(device)]
        return cls(kv_heads, s, head_dim, *parts)


def qattn_prefill_q8kv(q, cache: Q8KVCache, causal: bool = True, scale: float | None = None, out=None,
                       stream=None):
    """Attention of fp16 queries q [H, M, D] over a Q8_0 KV cache; returns fp16 [H, M, D]."""
    torch = _torch()
    if q.dtype != torch.float16 or not q.is_cuda or q.dim() != 3 or q.shape[2] != cache.head_dim:
        raise ValueError("q must be a float16 [H, M, D] tensor on a HIP device with D matching the cache")
    for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales):
        if t.device != q.device:
            raise ValueError(f"the KV cache is on {t.device}, the queries on {q.device}")
    q = q.contiguous()
    heads, m, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if m == 0:                 # no queries: nothing to launch (the C-ABI takes M >= 1)
        _check_out_device(out, q.device)
        if out.shape != q.shape:
            raise ValueError("out must be shaped like q")
        return out
    _check_out_device(out, q.device)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float16 tensor shaped like q")
    sc = float(scale) if scale is not None else 1.0 / math.sqrt(d)
    _check(lib().qattn_prefill_q8kv(q.data_ptr(), out.data_ptr(), heads, m, d, cache.k_codes.data_ptr(),
                                    cache.k_scales.data_ptr(), cache.v_codes.data_ptr(), cache.v_scales.data_ptr(),
                                    cache.kv_heads, cache.s, 1 if causal else 0, sc, _stream(stream)),
           "qattn_prefill_q8kv")
    return out


def qg_version() -> int:
    return int(lib().qg_version())
