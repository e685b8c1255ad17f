"""Host-side checks of libqgemm.so that need no GPU.

* The library loads and exports every function include/qgemm.h declares.
* qg_packed_sizes / qg_canonical_size follow the documented geometry.
* qg_pack_host moves bits only: reading the planar planes back with an
  independent reader written from the layout description gives, for every
  weight, the code and scale of the canonical bytes, hence the oracle's value.
* Argument errors come back as status codes before any launch (only rejected
  argument sets are used, so nothing reaches a device).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import quantized_prefill_gemm_codec_amd as qg
from golden_io import all_cases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = qg.lib()
    names = _header_functions()
    assert set(names) >= {"qgemm_prefill", "qgemm_swiglu", "qgemm_geglu", "qgemv_decode", "qg_pack_host", "qg_dequant"}
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(qg.EXPORTS)
    assert qg.qg_version() == 102


@pytest.mark.parametrize("codec,n,k", [(1, 8192, 2048), (1, 40, 96), (2, 14336, 4096), (3, 4096, 4096), (3, 33, 128),
                                     (4, 8192, 2048), (4, 40, 96), (5, 14336, 4096), (5, 33, 96),
                                     (6, 8192, 2048), (6, 40, 256), (7, 8192, 2048), (7, 40, 512),
                                     (8, 8192, 2048), (8, 40, 512)])
def test_sizes(codec, n, k):
    qs, sc = qg.qg_packed_sizes(codec, n, k)
    groups, ksteps = -(-n // 32), -(-k // 64)
    if codec == 7:
        assert qs == groups * ksteps * 416                    # 1.625 bits per weight of digits
    else:
        code_bytes = {1: 16, 2: 16, 3: 8, 4: 32, 5: 16, 6: 16, 8: 8}[codec]
        assert qs == groups * ksteps * 64 * code_bytes
    if codec in (1, 4):
        assert sc == groups * ksteps * 64 * 2
    elif codec == 2:
        assert sc == groups * ksteps * 32 * 4
    elif codec == 5:
        assert sc == groups * ksteps * 64 * 4
    elif codec == 6:
        assert sc == groups * (k // 256) * 640
    elif codec == 7:
        assert sc == groups * (k // 256) * 64
    else:
        assert sc == groups * (k // 128) * 32 * 2
    assert qg.qg_canonical_size(codec, n, k) == synth.canonical_bytes(codec, n, k)


def _ternary_digits(byte):
    """Digits (t0..t4, t0 most significant) of fixed-point base-3 bytes:
    byte = ceil(256 v / 243) inverts as v = floor(243 byte / 256)."""
    v = (np.asarray(byte, np.int64) * 243) // 256
    return np.stack([(v // 3 ** (4 - i)) % 3 for i in range(5)], axis=-1)


def _read_ternary_planar(n, k, qs, sc):
    groups, ksteps = -(-n // 32), -(-k // 64)
    ch = qs.reshape(groups, ksteps, 416)
    a = ch[:, :, :256].reshape(groups, ksteps, 64, 4)
    b = ch[:, :, 256:384].reshape(groups, ksteps, 64, 2)
    tail = ch[:, :, 384:].repeat(2, axis=2)                     # [groups, ksteps, 64]: byte of lane l // 2
    even = [_ternary_digits(x) for x in (a[..., 0], a[..., 2], b[..., 0])]
    odd = [_ternary_digits(x) for x in (a[..., 1], a[..., 3], b[..., 1])]
    td = _ternary_digits(tail)
    lane = np.arange(64)
    t = np.zeros((groups, ksteps, 64, 32), np.int64)
    for p in range(15):
        t[..., 2 * p] = even[p // 5][..., p % 5]
        t[..., 2 * p + 1] = odd[p // 5][..., p % 5]
    t[..., 30] = np.take_along_axis(td, (2 * (lane & 1))[None, None, :, None], axis=-1)[..., 0]
    t[..., 31] = np.take_along_axis(td, (2 * (lane & 1) + 1)[None, None, :, None], axis=-1)[..., 0]
    # lane 32 g + i: row 32 r + i, k = 64 t + 32 g + j
    codes = t.reshape(groups, ksteps, 2, 32, 32).transpose(0, 3, 1, 2, 4).reshape(groups * 32, ksteps * 64)
    codes = codes[:n, :k] - 1
    d = sc.view(np.float16).reshape(groups, k // 256, 32).astype(np.float64)
    rr, kk = np.arange(n), np.arange(k)
    scale = d[rr[:, None] // 32, kk[None, :] // 256, rr[:, None] % 32]
    return codes, scale, None


def _read_planar(codec, n, k, qs, sc):
    """Independent reader of the planar layout -> (codes [n,k], scale, bias)."""
    if codec == 7:
        return _read_ternary_planar(n, k, qs, sc)
    groups, ksteps = -(-n // 32), -(-k // 64)
    cb = {1: 16, 2: 16, 3: 8, 4: 32, 5: 16, 6: 16, 8: 8}[codec]
    if codec == 4:
        halves = qs.reshape(groups, ksteps, 2, 64, 16)
    else:
        lanes = qs.reshape(groups, ksteps, 64, cb)
    codes = np.zeros((groups * 32, ksteps * 64), np.int64)
    for j in range(32):
        if codec == 4:
            # dword 2 s + h' (h' = e // 4) of the lane; dwords 4 h .. 4 h + 3 in half h
            word = 2 * (j // 8) + (j % 8) // 4
            e4 = (j % 8) % 4
            bit = 8 * (e4 // 2) + 16 * (e4 % 2)
            q = halves[:, :, word // 4, :, (word % 4) * 4 + bit // 8].astype(np.int64) - 128
        elif codec in (3, 8):
            dw, e = divmod(j, 16)
            bit = 2 * (e // 2) + 16 * (e % 2)
            byte = lanes[..., 4 * dw + bit // 8].astype(np.int64)
            q = (byte >> (bit % 8)) & 3
        else:
            dw, e = divmod(j, 8)
            bit = 4 * (e // 2) + 16 * (e % 2)
            byte = lanes[..., 4 * dw + bit // 8].astype(np.int64)
            q = (byte >> (bit % 8)) & 15
        # q: [groups, ksteps, 64 lanes]; lane l = 32 g + i owns row 32 r + i, k = 64 t + 32 g + j
        for g in range(2):
            blk = q[:, :, 32 * g:32 * g + 32]                 # [groups, ksteps, 32 rows]
            rows = blk.transpose(0, 2, 1).reshape(groups * 32, ksteps)
            codes[:, np.arange(ksteps) * 64 + 32 * g + j] = rows
    codes = codes[:n, :k]
    kk = np.arange(k)
    rr = np.arange(n)
    if codec in (1, 4):
        d = sc.view(np.float16).reshape(groups, ksteps, 2, 32)
        blk = kk // 32
        scale = d[rr[:, None] // 32, blk[None, :] // 2, blk[None, :] % 2, rr[:, None] % 32]
        return codes, scale.astype(np.float64), None
    if codec == 6:
        # [groups][K/256][640 B]: u16 [4 k-steps][64 lanes] (sc, m bytes), then u32 [32 rows] (d, dmin)
        rec = sc.reshape(groups, k // 256, 640)
        scm = rec[:, :, :512].reshape(groups, k // 256, 4, 2, 32, 2).astype(np.int64)
        dd = rec[:, :, 512:].copy().view(np.float16).reshape(groups, k // 256, 32, 2).astype(np.float64)
        sub = kk // 32                                          # sub-block index along K
        sbk, u, gh = sub // 8, (sub % 8) // 2, sub % 2
        ri, rr32 = rr[:, None] // 32, rr[:, None] % 32
        scv = scm[ri, sbk[None, :], u[None, :], gh[None, :], rr32, 0]
        mv = scm[ri, sbk[None, :], u[None, :], gh[None, :], rr32, 1]
        d = dd[ri, sbk[None, :], rr32, 0]
        dmin = dd[ri, sbk[None, :], rr32, 1]
        return codes, d * scv, -(dmin * mv)
    if codec == 5:
        sb = sc.view(np.float16).reshape(groups, ksteps, 2, 32, 2)
        grp = kk // 32
        s = sb[rr[:, None] // 32, grp[None, :] // 2, grp[None, :] % 2, rr[:, None] % 32, 0]
        b = sb[rr[:, None] // 32, grp[None, :] // 2, grp[None, :] % 2, rr[:, None] % 32, 1]
        return codes, s.astype(np.float64), b.astype(np.float64)
    if codec == 2:
        sb = sc.view(np.float16).reshape(groups, ksteps, 32, 2)
        s = sb[rr[:, None] // 32, kk[None, :] // 64, rr[:, None] % 32, 0]
        b = sb[rr[:, None] // 32, kk[None, :] // 64, rr[:, None] % 32, 1]
        return codes, s.astype(np.float64), b.astype(np.float64)
    d = sc.view(np.float16).reshape(groups, k // 128, 32)
    scale = d[rr[:, None] // 32, kk[None, :] // 128, rr[:, None] % 32]
    return codes, scale.astype(np.float64), None     # Q2_0 and the 2-bit ternary layout: w = (q - 1) d


def _value(codec, codes, scale, bias):
    if codec == 1:
        return (codes - 8) * scale
    if codec in (4, 7):
        return codes * scale
    if codec in (2, 5, 6):
        return codes * scale + bias
    return (codes - 1) * scale


@pytest.mark.parametrize("codec,n,k", [(1, 40, 96), (1, 64, 64), (2, 33, 192), (3, 37, 256), (3, 32, 128),
                                     (4, 40, 96), (4, 64, 128), (5, 33, 96), (5, 64, 256), (6, 40, 512),
                                     (6, 64, 256), (7, 40, 512), (7, 64, 256), (7, 33, 768), (8, 40, 512),
                                     (8, 64, 256), (8, 33, 768)])
def test_pack_roundtrip_random(codec, n, k):
    canon = synth.gen_weight(codec, n, k, 77)
    qs, sc = qg.qg_pack_host(codec, n, k, canon)
    codes, scale, bias = _read_planar(codec, n, k, qs, sc)
    assert np.array_equal(_value(codec, codes, scale, bias), oracle.decode(codec, canon, n, k))


CASES = all_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_pack_roundtrip_golden(case):
    codec, n, k = case["codec"], case["n"], case["k"]
    canon = np.array(case["bytes"], np.uint8)
    qs, sc = qg.qg_pack_host(codec, n, k, canon)
    codes, scale, bias = _read_planar(codec, n, k, qs, sc)
    want = np.array(case["expect"], np.float64).reshape(n, k)
    assert np.array_equal(_value(codec, codes, scale, bias), want)


def test_pack_padding_decodes_to_zero():
    codec, n, k = 1, 40, 96       # N padded to 64 rows, K to 128
    qs, sc = qg.qg_pack_host(codec, n, k, synth.gen_weight(codec, n, k, 5))
    d = sc.view(np.float16).reshape(2, 2, 2, 32)
    assert np.all(d[1, :, :, 8:] == 0)          # rows 40..63
    assert np.all(d[:, 1, 1, :] == 0)           # k 96..127 (block 3)


def test_ternary_q2_layout_is_the_q2_0_layout():
    """The 2-bit ternary layout is the Q2_0 planar format of codes q = t: a
    Q2_0 matrix built from the same digits and scales packs to the same bytes
    (each 256-weight block's d written for both of its 128-weight halves)."""
    n, k = 45, 512
    rng = np.random.default_rng(8)
    t = rng.integers(0, 3, (n, k))
    d = synth.fp16_uniform(rng, 0.01, 0.03, (n, k // 256))
    q8 = qg.qg_pack_host(8, n, k, synth.encode_ternary((t - 1).astype(np.int8), d))
    q3 = qg.qg_pack_host(3, n, k, synth.encode_q2_0(t.astype(np.uint8), np.repeat(d, 2, axis=1)))
    assert np.array_equal(q8[0], q3[0]) and np.array_equal(q8[1], q3[1])
    assert qg.qg_kernel_for("prefill", 8, 2048, 8192, 2048) == qg.qg_kernel_for("prefill", 3, 2048, 8192, 2048)
    assert qg.qg_kernel_for("gemv", 8, 1, 14336, 4096) == "gemv_kernel<3, 1>"


def test_pack_rejects_invalid_ternary_bytes():
    canon = synth.gen_weight(7, 4, 256, 3)
    canon[54 + 2 + 17] = 243                                 # row 1, a five-digit byte
    qs = np.full(qg.qg_packed_sizes(7, 4, 256)[0], 0xAB, np.uint8)
    L = qg.lib()
    sc = np.zeros(qg.qg_packed_sizes(7, 4, 256)[1], np.uint8)
    assert L.qg_pack_host(7, 4, 256, canon.ctypes.data, canon.size, qs.ctypes.data, sc.ctypes.data) == -8
    assert np.all(qs == 0xAB)                                # nothing written
    canon[54 + 2 + 17] = 0
    canon[53] = 3                                            # the one-digit byte
    assert L.qg_pack_host(7, 4, 256, canon.ctypes.data, canon.size, qs.ctypes.data, sc.ctypes.data) == -8


def test_pack_errors():
    buf = np.zeros(64, np.uint8)
    L = qg.lib()
    p = buf.ctypes.data
    assert L.qg_pack_host(9, 1, 32, p, 64, p, p) == -2
    assert L.qg_pack_host(1, 1, 48, p, 64, p, p) == -3
    assert L.qg_pack_host(3, 1, 64, p, 64, p, p) == -3
    assert L.qg_pack_host(1, 0, 32, p, 64, p, p) == -3
    assert L.qg_pack_host(1, 2, 32, p, 35, p, p) == -7
    assert L.qg_pack_host(1, 1, 32, None, 64, p, p) == -1
    with pytest.raises(qg.QGError):
        qg.qg_packed_sizes(2, 4, 96)


def _w(codec=1, n=64, k=64, qs=0x10000, sc=0x20000, flags=0):
    return qg.qg_weight(codec, flags, n, k, qs, sc)


FAKE = 0x100000    # aligned, non-null; never dereferenced: every call below is rejected


@pytest.mark.parametrize("args,status", [
    (dict(w=_w(codec=9)), -2),
    (dict(w=_w(k=48)), -3),
    (dict(w=_w(flags=1)), -3),
    (dict(w=_w(qs=0)), -1),
    (dict(w=_w(qs=0x10008)), -4),
    (dict(m=0), -3),
    (dict(ldx=60), -3),
    (dict(ldx=68), -4),
    (dict(ldy=12), -3),
    (dict(x=FAKE + 8), -4),
    (dict(x=0), -1),
    (dict(y=0), -1),
])
def test_gemm_argument_errors(args, status):
    L = qg.lib()
    w = args.get("w", _w())
    m = args.get("m", 4)
    x = args.get("x", FAKE)
    y = args.get("y", FAKE)
    ldx = args.get("ldx", 64)
    ldy = args.get("ldy", 64)
    assert L.qgemm_prefill(ctypes.byref(w), x, m, ldx, y, ldy, None) == status
    assert L.qgemv_decode(ctypes.byref(w), x, m, ldx, y, ldy, None) == status
    assert L.qgemm_swiglu(ctypes.byref(w), ctypes.byref(w), x, m, ldx, y, ldy, None) == status
    assert L.qgemm_geglu(ctypes.byref(w), ctypes.byref(w), x, m, ldx, y, ldy, None) == status


def test_gemv_rejects_large_m_and_swiglu_mismatch():
    L = qg.lib()
    w = _w()
    assert L.qgemv_decode(ctypes.byref(w), FAKE, 65, 64, FAKE, 64, None) == -3
    pairs = [(_w(), _w(n=96)), (_w(), _w(k=128)), (_w(k=128), _w(codec=3, k=128))]
    for wg, wu in pairs:
        assert (wg.codec, wg.n, wg.k) != (wu.codec, wu.n, wu.k)
        assert L.qgemm_swiglu(ctypes.byref(wg), ctypes.byref(wu), FAKE, 4, wg.k, FAKE, 128, None) == -5
        assert L.qgemm_geglu(ctypes.byref(wg), ctypes.byref(wu), FAKE, 4, wg.k, FAKE, 128, None) == -5
    assert L.qg_dequant(ctypes.byref(_w()), FAKE, 60, None) == -3
    assert L.qg_dequant(ctypes.byref(_w(codec=0)), FAKE, 64, None) == -2


def test_prefill_heads_argument_errors():
    L = qg.lib()
    w = _w(n=128)
    for head_dim in (0, 4, 12, 48, 256):        # not a multiple of 8, or not dividing N = 128
        assert L.qgemm_prefill_heads(ctypes.byref(w), FAKE, 4, 64, FAKE, head_dim, None) == -3
    assert L.qgemm_prefill_heads(ctypes.byref(w), 0, 4, 64, FAKE, 64, None) == -1
    assert L.qgemm_prefill_heads(ctypes.byref(_w(codec=9)), FAKE, 4, 64, FAKE, 64, None) == -2
    assert L.qgemm_prefill_heads(ctypes.byref(w), FAKE + 8, 4, 64, FAKE, 64, None) == -4


def test_ternary_digit_identity_in_16_bit_arithmetic():
    """The kernels take digit i of a fixed-point base-3 byte B as
    X_(i+1) - 3 X_i with X_j = floor(B 3^j / 256), in 16-bit lanes; that equals
    ((B 3^i) mod 256) * 3 >> 8 for every valid byte, no product overflows 16
    bits, and the digits reproduce the byte's base-3 value."""
    for v in range(243):
        b = -(-256 * v // 243)                  # byte = ceil(256 v / 243)
        x = [((b * 3 ** j) & 0xFFFF) >> 8 for j in range(6)]
        assert all(b * 3 ** j < 1 << 16 for j in range(6))
        digits = [(x[i + 1] - 3 * x[i]) & 0xFFFF for i in range(5)]
        assert digits == [((b * 3 ** i) & 0xFF) * 3 >> 8 for i in range(5)]
        assert sum(t * 3 ** (4 - i) for i, t in enumerate(digits)) == v


def test_stream_read_argument_errors():
    L = qg.lib()
    assert L.qg_stream_read(0, 1024, FAKE, None) == -1
    assert L.qg_stream_read(FAKE, 1024, 0, None) == -1
    for nbytes in (0, 8, 1000, 1 << 31):
        assert L.qg_stream_read(FAKE, nbytes, FAKE, None) == -3
    assert L.qg_stream_read(FAKE + 8, 1024, FAKE, None) == -4
    assert L.qg_stream_read(FAKE, 1024, FAKE + 4, None) == -4


def test_status_strings():
    for st in qg.STATUS:
        assert qg.lib().qg_status_str(st)


def test_pack_kv_host_splits_blocks():
    rows, d = 5, 128
    canon = synth.gen_q8_0(rows, d, 31)
    L = qg.lib()
    codes = np.empty(rows * d, np.uint8)
    scales = np.empty(rows * (d // 32) * 2, np.uint8)
    assert L.qg_pack_kv_host(canon.ctypes.data, canon.size, rows, d, codes.ctypes.data, scales.ctypes.data) == 0
    blk = canon.reshape(rows, d // 32, 34)
    assert np.array_equal(scales.reshape(rows, d // 32, 2), blk[:, :, :2])
    assert np.array_equal(codes.reshape(rows, d // 32, 32), blk[:, :, 2:] ^ 0x80)     # q + 128
    # decoded from the planar split, the values are the oracle's Q8_0 decode
    w = (codes.reshape(rows, d).astype(np.float64) - 128.0) * np.repeat(
        scales.view(np.float16).reshape(rows, d // 32).astype(np.float64), 32, axis=1)
    assert np.array_equal(w, oracle.decode(oracle.Q8_0, canon, rows, d))
    assert L.qg_pack_kv_host(canon.ctypes.data, canon.size - 1, rows, d, codes.ctypes.data, scales.ctypes.data) == -7
    assert L.qg_pack_kv_host(canon.ctypes.data, canon.size, rows, 48, codes.ctypes.data, scales.ctypes.data) == -3
    assert L.qg_pack_kv_host(0, canon.size, rows, d, codes.ctypes.data, scales.ctypes.data) == -1


def _attn(L, **kw):
    a = dict(q=FAKE, o=FAKE, heads=4, m=8, d=64, kq=FAKE, ks=FAKE, vq=FAKE, vs=FAKE, kvh=2, s=8, causal=1, scale=0.125)
    a.update(kw)
    return L.qattn_prefill_q8kv(a["q"], a["o"], a["heads"], a["m"], a["d"], a["kq"], a["ks"], a["vq"], a["vs"],
                                a["kvh"], a["s"], a["causal"], a["scale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(vs=0), -1), (dict(d=96), -3), (dict(d=32), -3), (dict(kvh=3), -3), (dict(heads=0), -3),
    (dict(m=0), -3), (dict(s=7), -3), (dict(causal=2), -3), (dict(scale=0.0), -3), (dict(scale=float("nan")), -3),
    (dict(scale=float("inf")), -3), (dict(heads=70000, kvh=1), -3), (dict(q=FAKE + 2), -4), (dict(ks=FAKE + 8), -4),
])
def test_attention_argument_errors(kw, status):
    assert _attn(qg.lib(), **kw) == status


def test_build_guard_rejects_kernels_with_scratch_or_spills():
    """The build parses hipcc's resource-usage remarks and refuses a library
    whose kernels spill registers to scratch or exceed the compute unit's LDS;
    the remark format it reads is the compiler's."""
    from quantized_prefill_gemm_codec_amd import build as qbuild

    def remarks(name, scratch, vspill, lds):
        pre = "x.hip:1:1: remark: "
        tail = " [-Rpass-analysis=kernel-resource-usage]"
        return "\n".join([pre + f"Function Name: {name}" + tail, pre + "    VGPRs: 128" + tail,
                          pre + "    AGPRs: 0" + tail, pre + f"    ScratchSize [bytes/lane]: {scratch}" + tail,
                          pre + "    Dynamic Stack: False" + tail, pre + "    Occupancy [waves/SIMD]: 2" + tail,
                          pre + "    SGPRs Spill: 0" + tail, pre + f"    VGPRs Spill: {vspill}" + tail,
                          pre + f"    LDS Size [bytes/block]: {lds}" + tail])

    ok = qbuild.kernel_resources(remarks("_Z2okv", 0, 0, 65536))
    assert ok["_Z2okv"]["ScratchSize [bytes/lane]"] == "0"
    assert len(qbuild.check_resources(ok)) == 1
    for bad in (remarks("_Z3badv", 16, 0, 1024), remarks("_Z3badv", 0, 3, 1024), remarks("_Z3badv", 0, 0, 200000)):
        with pytest.raises(RuntimeError, match="over their resource budget"):
            qbuild.check_resources(qbuild.kernel_resources(bad))


def test_built_kernels_use_no_scratch():
    """The table the last build wrote: every kernel without scratch or spills."""
    from quantized_prefill_gemm_codec_amd import build as qbuild
    if not os.path.exists(qbuild.RESOURCES):
        pytest.skip("library not built in this tree")
    lines = open(qbuild.RESOURCES).read().splitlines()
    assert len(lines) >= 80
    assert all(" scratch=0 spills=0 " in ln for ln in lines), [ln for ln in lines if " scratch=0 spills=0 " not in ln]


def test_build_guard_rejects_q4_k_double_rounding():
    """The build disassembles the device code and refuses a Q4_K unpacking
    kernel whose fused multiply-add is narrowed to fp16 by a separate
    conversion (two roundings) instead of v_fma_mixlo/hi_f16 (one)."""
    from quantized_prefill_gemm_codec_amd import build as qbuild
    name = "_ZN2qg12_GLOBAL__N_115gemm_dma_kernelILi6ELi64ELi64EEEvv"
    once = (f"0000000000001000 <{name}>:\n\tv_fma_mixlo_f16 v1, v2, v3, v4 // 000000001000: D3A10001\n"
            "\tv_fma_mixhi_f16 v1, v2, v3, v4\n\tv_mfma_f32_32x32x16_f16 v[0:15], v[1:4], v[5:8], v[0:15]\n"
            "0000000000002000 <_ZN2qg12_GLOBAL__N_115gemm_dma_kernelILi1ELi64ELi64EEEvv>:\n\tv_pk_mul_f16 v1, v2, v3\n")
    funcs = qbuild.parse_disassembly(once)
    assert funcs[name] == {"v_fma_mixlo_f16": 1, "v_fma_mixhi_f16": 1, "v_mfma_f32_32x32x16_f16": 1}
    assert len(qbuild.check_single_rounding(funcs)) == 1        # the Q4_0 kernel is not checked
    twice = once.replace("v_fma_mixhi_f16 v1, v2, v3, v4", "v_fma_mix_f32 v5, v2, v3, v4\n\tv_cvt_pk_f16_f32 v1, v5, v6")
    with pytest.raises(RuntimeError, match="may round twice"):
        qbuild.check_single_rounding(qbuild.parse_disassembly(twice))
    with pytest.raises(RuntimeError, match="no Q4_K"):
        qbuild.check_single_rounding({})


def test_built_q4_k_kernels_round_once():
    """The table the last build wrote: every Q4_K unpacking kernel (the GEMM
    tiles and the dequant kernel) narrows with v_fma_mixlo/hi_f16 only."""
    from quantized_prefill_gemm_codec_amd import build as qbuild
    if not os.path.exists(qbuild.ROUNDING):
        pytest.skip("library not built in this tree")
    lines = open(qbuild.ROUNDING).read().splitlines()
    assert len(lines) >= 8
    assert any("dequant_kernel" in ln for ln in lines)
    for ln in lines:
        counts = dict(kv.split("=") for kv in ln.rsplit(": ", 1)[1].split())
        assert int(counts["v_fma_mixlo_f16"]) > 0 and int(counts["v_fma_mixhi_f16"]) > 0, ln
        assert int(counts["v_fma_mix_f32"]) == 0, ln


def test_pack_is_reentrant_across_threads():
    """The library keeps no state: the host repack called from many threads at
    once gives every caller the planes a lone call gives."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(codec, 64 + 32 * (codec % 3), 256 * (1 + codec % 2)) for codec in range(1, 9)] * 3
    canon = {j: synth.gen_weight(j[0], j[1], j[2], 500 + j[0]) for j in set(jobs)}
    alone = {j: qg.qg_pack_host(*j, canon[j]) for j in set(jobs)}
    with ThreadPoolExecutor(8) as ex:
        results = list(ex.map(lambda j: (j, qg.qg_pack_host(*j, canon[j])), jobs))
    for j, (qs, sc) in results:
        assert np.array_equal(qs, alone[j][0]) and np.array_equal(sc, alone[j][1])
