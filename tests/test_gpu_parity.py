"""GPU parity of the HIP path against the fp64 oracle, through the C-ABI.

Bars (the method's own): dequantized fp16 weights bit-exact against the
oracle's correctly rounded decode; GEMM / SwiGLU / GEMV outputs finite and
within max|err| / rms(ref) <= 1e-2 of the fp64 reference.  Full-size workloads
are checked on sampled rows and columns the oracle computes directly.
Integer-exact properties (identity probe, power-of-two scaling, row
permutation, run-to-run determinism) are checked bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
import quantized_prefill_gemm_codec_amd as qg

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no HIP device")
    return t


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _weight(torch, codec, n, k, canon):
    return qg.QWeight.from_canonical(codec, n, k, canon, device="cuda")


def _err(y, ref):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(y - ref)) / rms)


def _err_beyond_fp16_rounding(y, ref):
    """max over elements of (|y - ref| - 2^-11 |ref|) / rms(ref).

    The fused SwiGLU output is fp16 and heavy-tailed (a product of two
    near-Gaussian sums): the half-ulp rounding of the output format alone,
    up to 2^-11 |ref|, reaches ~1e-2 of rms at the largest elements.  The
    tolerance applies to the error on top of that unavoidable rounding.
    """
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.maximum(np.abs(y - ref) - 2.0 ** -11 * np.abs(ref), 0.0)) / rms)


def _same_value_bits(a16, b16):
    """fp16 arrays equal bit for bit, except that +0 and -0 compare equal."""
    a = np.asarray(a16).view(np.uint16)
    b = np.asarray(b16).view(np.uint16)
    zero = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)
    return bool(np.all((a == b) | zero))


# ------------------------------------------------------------- dequantization --

DEQ_SHAPES = [(1, 256, 256), (1, 40, 96), (1, 1000, 544), (2, 33, 192), (2, 300, 1024),
              (3, 37, 256), (3, 520, 1152), (4, 256, 256), (4, 40, 96), (4, 300, 544),
              (5, 256, 256), (5, 33, 96), (5, 300, 544), (6, 256, 256), (6, 40, 512), (6, 300, 768),
              (7, 256, 256), (7, 40, 512), (7, 300, 768), (8, 256, 256), (8, 40, 512), (8, 300, 768)]


@pytest.mark.parametrize("codec,n,k", DEQ_SHAPES)
def test_dequant_bit_exact(torch, codec, n, k):
    canon = synth.gen_weight(codec, n, k, 1000 + n)
    w = _weight(torch, codec, n, k, canon)
    got = qg.qg_dequant(w).cpu().numpy()
    want = oracle.dequant_f16_bits(codec, canon, n, k).view(np.float16)
    assert _same_value_bits(got, want)


def test_dequant_keeps_subnormal_bias(torch):
    n, k = 32, 128
    codes = np.zeros((n, k), np.uint8)
    s = np.full((n, k // 64), 0.5, np.float16)
    b = (np.arange(n * (k // 64)).reshape(n, k // 64) % 7 + 1).astype(np.uint16).view(np.float16)   # subnormals
    canon = synth.encode_mlx4(codes, s, b)
    got = qg.qg_dequant(_weight(torch, 2, n, k, canon)).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), np.repeat(b.view(np.uint16), 64, axis=1))


def test_dequant_q4_k_extreme_scales(torch):
    """d and dmin from the largest normal to the smallest subnormal binary16:
    every weight is the correctly rounded fp16 of d sc q - dmin m (one rounding)."""
    pats = np.array([0x7BFF, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x3555, 0xFBFF, 0x8001, 0x1234, 0x6A5A], np.uint16)
    pairs = [(a, b) for a in pats for b in pats]
    n, k = len(pairs), 512
    rng = np.random.default_rng(61)
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    sc = rng.integers(0, 64, (n, k // 32)).astype(np.uint8)
    mn = rng.integers(0, 64, (n, k // 32)).astype(np.uint8)
    d = np.repeat(np.array([a for a, _ in pairs], np.uint16).view(np.float16)[:, None], 2, axis=1)
    dmin = np.repeat(np.array([b for _, b in pairs], np.uint16).view(np.float16)[:, None], 2, axis=1)
    canon = synth.encode_q4_k(codes, sc, mn, d, dmin)
    got = qg.qg_dequant(_weight(torch, 6, n, k, canon)).cpu().numpy()
    want = oracle.dequant_f16_bits(6, canon, n, k).view(np.float16)
    assert _same_value_bits(got, want)


def _q4_k_tie_weights(n, k):
    """d = 1 + 2^-10 and a tiny dmin: d sc q lands exactly halfway between two
    binary16 values whenever sc q = 3 * 2^j, and -dmin m moves it just off the
    tie.  One rounding of the exact value and a detour through fp32 (which
    drops the tiny term, then rounds the tie to even) disagree there."""
    rng = np.random.default_rng(62)
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    sc = rng.integers(0, 64, (n, k // 32)).astype(np.uint8)
    mn = rng.integers(1, 64, (n, k // 32)).astype(np.uint8)
    d = np.full((n, k // 256), 0x3C01, np.uint16).view(np.float16)
    dmin = np.where(np.arange(n)[:, None] % 2 == 0, 0x0001, 0x8001).astype(np.uint16)
    dmin = np.repeat(dmin, k // 256, axis=1).view(np.float16)
    return synth.encode_q4_k(codes, sc, mn, d, dmin)


def test_q4_k_single_rounding_through_kernels(torch):
    n = k = 256
    canon = _q4_k_tie_weights(n, k)
    want = oracle.dequant_f16_bits(6, canon, n, k).view(np.float16)
    w = _weight(torch, 6, n, k, canon)
    assert _same_value_bits(qg.qg_dequant(w).cpu().numpy(), want)
    eye = torch.eye(k, dtype=torch.float16, device="cuda")
    for m in (256, 128):      # the 128-row prefill tile, the split-k 64 x 64 tile
        y = qg.qgemm_prefill(w, eye[:m].contiguous()).cpu().numpy()
        assert _same_value_bits(y, want.T[:m])


def test_q4_k_single_rounding_through_the_wide_tile(torch):
    """The same tie weights through the 128 x 512 prefill tile, which only a
    grid of 256 or more tiles reaches: X is the identity repeated 16 times."""
    n, k, reps = 4096, 256, 16
    assert qg.qg_kernel_for("prefill", 6, reps * k, n, k) == "gemm_dma_kernel<6, 128, 512, 1, 8, 1, 0, 3, 1>"
    canon = _q4_k_tie_weights(n, k)
    want = oracle.dequant_f16_bits(6, canon, n, k).view(np.float16)
    w = _weight(torch, 6, n, k, canon)
    eye = torch.eye(k, dtype=torch.float16, device="cuda").repeat(reps, 1).contiguous()
    y = qg.qgemm_prefill(w, eye).cpu().numpy()
    for r in (0, 7, reps - 1):
        assert _same_value_bits(y[r * k:(r + 1) * k], want.T)


@pytest.mark.parametrize("codec", [1, 2, 3, 4, 5, 6, 7, 8])
def test_identity_probe_through_gemm(torch, codec):
    """X = I: every output is one product with 1.0, so Y = W^T exactly."""
    n = k = 256
    canon = synth.gen_weight(codec, n, k, 2000 + codec)
    w = _weight(torch, codec, n, k, canon)
    x = torch.eye(k, dtype=torch.float16, device="cuda")
    y = qg.qgemm_prefill(w, x).cpu().numpy()
    want = oracle.dequant_f16_bits(codec, canon, n, k).view(np.float16).T
    assert _same_value_bits(y, want)


# --------------------------------------------------------------- prefill GEMM --

GEMM_SHAPES = [
    (1, 16, 256, 256), (1, 5, 200, 96), (1, 33, 256, 288), (1, 127, 520, 64), (1, 128, 256, 32),
    (1, 129, 136, 160), (1, 300, 264, 352), (1, 257, 1024, 256),
    (2, 6, 256, 192), (2, 65, 200, 64), (2, 129, 272, 320), (2, 300, 512, 256),
    (3, 7, 96, 128), (3, 100, 264, 384), (3, 129, 256, 256), (3, 320, 520, 512),
    # small M with several k-steps per slice of the split k-loop, ragged last slice
    (1, 48, 320, 2080), (2, 40, 72, 1152), (3, 64, 96, 1408),
    # Q8_0 through every kernel shape class
    (4, 16, 256, 256), (4, 33, 200, 288), (4, 129, 136, 160), (4, 300, 264, 352), (4, 257, 1024, 256),
    # MLX4-G32 likewise
    (5, 16, 256, 256), (5, 33, 200, 288), (5, 129, 136, 160), (5, 300, 264, 352), (5, 257, 1024, 256),
    # Q4_K likewise (K a multiple of the 256-weight super-block), and a split-k shape
    (6, 16, 256, 256), (6, 33, 200, 512), (6, 129, 136, 256), (6, 300, 264, 768), (6, 257, 1024, 256),
    (6, 48, 320, 2304),
    # ternary likewise, plus two 64-row tiles of the split-k small-M tile (64 < M <= 128)
    (7, 16, 256, 256), (7, 33, 200, 512), (7, 100, 136, 256), (7, 129, 136, 256), (7, 300, 264, 768),
    (7, 257, 1024, 256), (7, 48, 320, 2304), (6, 100, 264, 512),
    # two 64-row tiles of the split-k small-M tile for the remaining codecs
    (2, 100, 200, 256), (4, 100, 200, 256), (5, 96, 136, 288),
]


@pytest.mark.parametrize("codec,m,n,k", GEMM_SHAPES)
def test_prefill_parity(torch, codec, m, n, k):
    seed = 3000 + m + n + k
    canon = synth.gen_weight(codec, n, k, seed)
    x = synth.gen_x(m, k, seed)
    w = _weight(torch, codec, n, k, canon)
    y = qg.qgemm_prefill(w, _dev(torch, x)).cpu().numpy()
    ref = oracle.gemm_ref(codec, canon, n, k, x)
    assert _err(y, ref) <= TOL


def test_prefill_leading_dims_and_strides(torch):
    codec, n, k = 1, 136, 192
    canon = synth.gen_weight(codec, n, k, 41)
    w = _weight(torch, codec, n, k, canon)
    x = synth.gen_x(6, k, 42)
    ref = oracle.gemm_ref(codec, canon, n, k, x)
    y3 = qg.qgemm_prefill(w, _dev(torch, x).reshape(2, 3, k)).cpu().numpy()
    assert y3.shape == (2, 3, n) and _err(y3.reshape(6, n), ref) <= TOL
    wide = torch.zeros((6, k + 40), dtype=torch.float16, device="cuda")
    wide[:, :k] = _dev(torch, x)
    wide[:, k:] = float("nan")                       # must never be read
    out = torch.full((6, n + 24), float("nan"), dtype=torch.float16, device="cuda")
    qg.qgemm_prefill(w, wide[:, :k], out=out[:, :n])
    o = out.cpu().numpy()
    assert _err(o[:, :n], ref) <= TOL
    assert np.all(np.isnan(o[:, n:].astype(np.float32)))   # columns past N untouched


def test_prefill_power_of_two_scale_is_exact(torch):
    codec, m, n, k = 1, 300, 256, 256
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    d = rng.uniform(0.005, 0.02, (n, k // 32)).astype(np.float16)
    x = _dev(torch, synth.gen_x(m, k, 6))
    y1 = qg.qgemm_prefill(_weight(torch, codec, n, k, synth.encode_q4_0(codes, d)), x).cpu().numpy()
    y2 = qg.qgemm_prefill(_weight(torch, codec, n, k, synth.encode_q4_0(codes, d * np.float16(2))), x).cpu().numpy()
    a, b = y1.astype(np.float64), y2.astype(np.float64)
    # x2 commutes with every fp32 rounding and with the fp16 output rounding,
    # except in the fp16 subnormal range, whose quantum is fixed at 2^-24
    normal = np.abs(a) >= 2.0 ** -14
    assert normal.mean() > 0.99
    bad = normal & (b != 2 * a)
    assert not bad.any(), (int(bad.sum()), a[bad][:5], b[bad][:5])
    assert np.all(np.abs(b - 2 * a)[~normal] <= 2.0 ** -23)


def test_prefill_row_permutation_and_determinism(torch):
    codec, m, n, k = 2, 512, 512, 512
    canon = synth.gen_weight(codec, n, k, 7)
    w = _weight(torch, codec, n, k, canon)
    x = synth.gen_x(m, k, 8)
    perm = np.random.default_rng(9).permutation(m)
    y = qg.qgemm_prefill(w, _dev(torch, x)).cpu().numpy()
    y_again = qg.qgemm_prefill(w, _dev(torch, x)).cpu().numpy()
    yp = qg.qgemm_prefill(w, _dev(torch, x[perm])).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), y_again.view(np.uint16))
    assert np.array_equal(yp.view(np.uint16), y[perm].view(np.uint16))


HEADS_SHAPES = [(1, 2, 256, 128, 64), (2, 37, 192, 256, 64), (1, 300, 512, 256, 128), (3, 64, 384, 256, 96),
                (4, 129, 256, 160, 32), (6, 37, 192, 256, 64), (7, 300, 256, 512, 128),
                (1, 2048, 8192, 128, 128)]


@pytest.mark.parametrize("codec,m,n,k,d", HEADS_SHAPES)
def test_prefill_heads_layout(torch, codec, m, n, k, d):
    """[H, M, D] output is the row-major output with n = h D + d moved, bit for bit."""
    seed = 3500 + m + n + k
    canon = synth.gen_weight(codec, n, k, seed)
    x = synth.gen_x(m, k, seed)
    w = _weight(torch, codec, n, k, canon)
    xd = _dev(torch, x)
    yh = qg.qgemm_prefill_heads(w, xd, d).cpu().numpy()
    y = qg.qgemm_prefill(w, xd).cpu().numpy()
    assert yh.shape == (n // d, m, d)
    assert np.array_equal(yh.view(np.uint16), y.reshape(m, n // d, d).transpose(1, 0, 2).view(np.uint16))
    if m <= 300:
        ref = oracle.gemm_ref(codec, canon, n, k, x)
        assert _err(yh.transpose(1, 0, 2).reshape(m, n), ref) <= TOL


# -------------------------------------------------------------------- SwiGLU --

SWIGLU_SHAPES = [(2, 33, 200, 192), (2, 130, 256, 128), (2, 300, 264, 256), (1, 70, 136, 96), (3, 200, 128, 256),
                 (4, 200, 128, 256), (4, 70, 136, 96), (5, 200, 128, 256), (5, 70, 136, 96),
                 (6, 300, 264, 256), (6, 70, 136, 512), (7, 300, 264, 256), (7, 70, 136, 512),
                 (7, 40, 64, 256),
                 # the split-k small-M tile with both matrices: Q2_0 (64-byte scale records, two row
                 # groups per matrix), one and two 64-row tiles, ragged N and a K tail of 128
                 (3, 40, 72, 256), (3, 100, 136, 384), (1, 128, 200, 160)]


@pytest.mark.parametrize("codec,m,n,k", SWIGLU_SHAPES)
def test_swiglu_parity(torch, codec, m, n, k):
    seed = 4000 + m + n
    cg = synth.gen_weight(codec, n, k, seed, synth.T_WG)
    cu = synth.gen_weight(codec, n, k, seed, synth.T_WU)
    x = synth.gen_x(m, k, seed)
    y = qg.qgemm_swiglu(_weight(torch, codec, n, k, cg), _weight(torch, codec, n, k, cu), _dev(torch, x)).cpu().numpy()
    ref = oracle.swiglu_ref(codec, cg, cu, n, k, x)
    assert _err_beyond_fp16_rounding(y, ref) <= TOL


def test_swiglu_one_hot_probe(torch):
    """One-hot X rows and an up matrix of exact ones: out = SiLU(wg[n, k_m])."""
    m, n, k = 64, 256, 128
    cg = synth.gen_weight(2, n, k, 11, synth.T_WG)
    ones = synth.encode_mlx4(np.zeros((n, k), np.uint8), np.full((n, 2), 0.25, np.float16),
                             np.ones((n, 2), np.float16))
    km = np.arange(m) * 2 % k
    x = np.zeros((m, k), np.float16)
    x[np.arange(m), km] = 1
    y = qg.qgemm_swiglu(_weight(torch, 2, n, k, cg), _weight(torch, 2, n, k, ones), _dev(torch, x)).cpu().numpy()
    g = oracle.dequant_f16_bits(2, cg, n, k).view(np.float16).astype(np.float64)[:, km].T
    ref = oracle.swiglu(g, np.ones_like(g))
    assert np.all(np.abs(y.astype(np.float64) - ref) <= 2.0 ** -10 * np.abs(ref) + 2.0 ** -24)


# -------------------------------------------------------------------- GeGLU --

GEGLU_SHAPES = [(2, 300, 264, 256), (2, 70, 136, 128), (1, 33, 200, 192), (4, 200, 128, 256), (3, 129, 256, 256),
                (6, 129, 256, 256), (7, 129, 256, 256)]


@pytest.mark.parametrize("codec,m,n,k", GEGLU_SHAPES)
def test_geglu_parity(torch, codec, m, n, k):
    seed = 4500 + m + n
    cg = synth.gen_weight(codec, n, k, seed, synth.T_WG)
    cu = synth.gen_weight(codec, n, k, seed, synth.T_WU)
    x = synth.gen_x(m, k, seed)
    y = qg.qgemm_geglu(_weight(torch, codec, n, k, cg), _weight(torch, codec, n, k, cu), _dev(torch, x)).cpu().numpy()
    ref = oracle.geglu_ref(codec, cg, cu, n, k, x)
    assert _err_beyond_fp16_rounding(y, ref) <= TOL


def test_geglu_one_hot_probe(torch):
    """One-hot X rows and an up matrix of exact ones: out = GELU(wg[n, k_m])."""
    m, n, k = 64, 256, 128
    cg = synth.gen_weight(2, n, k, 12, synth.T_WG)
    ones = synth.encode_mlx4(np.zeros((n, k), np.uint8), np.full((n, 2), 0.25, np.float16),
                             np.ones((n, 2), np.float16))
    km = np.arange(m) * 2 % k
    x = np.zeros((m, k), np.float16)
    x[np.arange(m), km] = 1
    y = qg.qgemm_geglu(_weight(torch, 2, n, k, cg), _weight(torch, 2, n, k, ones), _dev(torch, x)).cpu().numpy()
    g = oracle.dequant_f16_bits(2, cg, n, k).view(np.float16).astype(np.float64)[:, km].T
    ref = oracle.geglu(g, np.ones_like(g))
    assert np.all(np.abs(y.astype(np.float64) - ref) <= 2.0 ** -10 * np.abs(ref) + 2.0 ** -24)


# ---------------------------------------------------------------------- GEMV --

GEMV_SHAPES = [(1, 1, 1000, 512), (1, 2, 256, 96), (1, 3, 520, 256), (1, 4, 200, 1024), (1, 5, 256, 256),
               (1, 17, 136, 192), (1, 64, 512, 512), (2, 1, 300, 256), (2, 4, 256, 512), (2, 33, 256, 128),
               (3, 1, 264, 512), (3, 3, 256, 256), (3, 64, 200, 384),
               (4, 1, 1000, 512), (4, 3, 264, 256), (4, 64, 200, 384),
               (5, 1, 1000, 512), (5, 2, 264, 96), (5, 64, 200, 384),
               (6, 1, 1000, 512), (6, 2, 256, 1024), (6, 3, 264, 256), (6, 64, 200, 512),
               (7, 1, 1000, 512), (7, 2, 256, 1024), (7, 4, 264, 256), (7, 64, 200, 512)]


@pytest.mark.parametrize("codec,m,n,k", GEMV_SHAPES)
def test_gemv_parity(torch, codec, m, n, k):
    seed = 5000 + m + n + k
    canon = synth.gen_weight(codec, n, k, seed)
    x = synth.gen_x(m, k, seed)
    w = _weight(torch, codec, n, k, canon)
    y = qg.qgemv_decode(w, _dev(torch, x)).cpu().numpy()
    ref = oracle.gemm_ref(codec, canon, n, k, x)
    assert _err(y, ref) <= TOL
    y2 = qg.qgemv_decode(w, _dev(torch, x)).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_gemv_single_vector_shape(torch):
    codec, n, k = 1, 256, 256
    canon = synth.gen_weight(codec, n, k, 51)
    x = synth.gen_x(1, k, 52)
    y = qg.qgemv_decode(_weight(torch, codec, n, k, canon), _dev(torch, x[0])).cpu().numpy()
    assert y.shape == (n,)
    assert _err(y[None, :], oracle.gemm_ref(codec, canon, n, k, x)) <= TOL


# ----------------------------------------------------- full-size workloads --

def _sample(rng, size, count):
    if size <= count:
        return np.arange(size)
    s = rng.choice(np.arange(1, size - 1), count - 2, replace=False)
    return np.sort(np.concatenate([[0, size - 1], s]))


@pytest.mark.parametrize("codec", [1, 2, 3, 4, 5, 6, 7, 8])
def test_prefill_wide_tile_ragged(torch, codec):
    """M = 1921, N = 7681 is 16 x 16 tiles of 128 x 512 (the tile the prefill
    takes when those fill the chip), with a one-row m tail and a one-column n
    tail inside a partly filled row group; sampled rows and columns include
    both tails."""
    m, n, k = 1921, 7681, 256
    canon = synth.gen_weight(codec, n, k, 4100 + codec)
    x = synth.gen_x(m, k, 4200 + codec)
    w = _weight(torch, codec, n, k, canon)
    y = qg.qgemm_prefill(w, _dev(torch, x))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    rng = np.random.default_rng(codec)
    rows_m = np.unique(np.concatenate([_sample(rng, m, 12), [1919, 1920]]))
    rows_n = np.unique(np.concatenate([_sample(rng, n, 384), np.arange(7664, 7681)]))
    ref = oracle.gemm_ref(codec, canon, n, k, x[rows_m], rows_n=rows_n)
    assert _err(y.cpu().numpy()[np.ix_(rows_m, rows_n)], ref) <= TOL


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_workload_sampled(torch, name):
    wl = synth.WORKLOADS[name]
    x = wl.x()
    mats = wl.weights()
    ws = [_weight(torch, wl.codec, wl.n, wl.k, c) for c in mats]
    xd = _dev(torch, x)
    if wl.op == "swiglu":
        y = qg.qgemm_swiglu(ws[0], ws[1], xd)
    elif wl.op == "geglu":
        y = qg.qgemm_geglu(ws[0], ws[1], xd)
    elif wl.op == "heads":
        y = qg.qgemm_prefill_heads(ws[0], xd, wl.head_dim).permute(1, 0, 2).reshape(wl.m, wl.n)
    elif wl.op == "gemv":
        y = qg.qgemv_decode(ws[0], xd)
    else:
        y = qg.qgemm_prefill(ws[0], xd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    rng = np.random.default_rng(wl.seed)
    rows_m = _sample(rng, wl.m, 12)
    rows_n = _sample(rng, wl.n, 384)
    ys = y.cpu().numpy()[np.ix_(rows_m, rows_n)]
    if wl.op in synth.GATED:
        fn = oracle.swiglu_ref if wl.op == "swiglu" else oracle.geglu_ref
        ref = fn(wl.codec, mats[0], mats[1], wl.n, wl.k, x[rows_m], rows_n=rows_n)
        assert _err_beyond_fp16_rounding(ys, ref) <= TOL
    else:
        ref = oracle.gemm_ref(wl.codec, mats[0], wl.n, wl.k, x[rows_m], rows_n=rows_n)
        assert _err(ys, ref) <= TOL


# ------------------------------------------------------- binding guards --

def test_out_that_needs_a_copy_is_rejected_before_launch(torch):
    """A caller's out that cannot be viewed as [M, N] rows (a strided 3-D
    slice), lives on the host, or on another device is rejected with
    ValueError and the buffer is left untouched: nothing is launched."""
    codec, n, k = 1, 64, 64
    canon = synth.gen_weight(codec, n, k, 71)
    w = _weight(torch, codec, n, k, canon)
    x = _dev(torch, synth.gen_x(6, k, 72)).reshape(2, 3, k)
    buf = torch.full((2, 4, n), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        qg.qgemm_prefill(w, x, out=buf[:, :3, :])
    torch.cuda.synchronize()
    assert bool((buf == 7.0).all())
    with pytest.raises(ValueError):
        qg.qgemm_prefill(w, x, out=torch.empty((2, 3, n), dtype=torch.float16))
    with pytest.raises(ValueError):
        qg.qgemm_prefill_heads(w, x.reshape(6, k), 32, out=torch.empty((2, 6, 32), dtype=torch.float16))
    with pytest.raises(ValueError):
        qg.qgemm_prefill(w, x, out=torch.empty((2, 3, n), dtype=torch.float32, device="cuda"))
    good = torch.empty((2, 3, n), dtype=torch.float16, device="cuda")
    assert qg.qgemm_prefill(w, x, out=good) is good
    assert _err(good.reshape(6, n).cpu().numpy(), oracle.gemm_ref(codec, canon, n, k, synth.gen_x(6, k, 72))) <= TOL


# ------------------------------------------------- non-finite tripwire --

def _poison_scale(codec, canon, n, k, row, block):
    """Canonical bytes with the fp16 scale (Q4_K: d) of one block of one row set to +Inf."""
    c = canon.copy()
    if codec in (2, 5):                                   # MLX: codes, then the fp16 scale plane
        g = 64 if codec == 2 else 32
        off = n * k // 2 + 2 * (row * (k // g) + block)
    else:                                                 # block structs that open with fp16 d
        size = {1: 18, 3: 34, 4: 34, 6: 144, 7: 54}[codec]
        off = (row * (k // synth.BLOCK[codec]) + block) * size
    c[off:off + 2] = np.array([0x7C00], np.uint16).view(np.uint8)
    return c


NONFINITE_CASES = [("prefill", 1, 300), ("prefill", 2, 33), ("prefill", 3, 1), ("prefill", 6, 129),
                   ("gemv", 1, 64), ("gemv", 4, 2), ("gemv", 7, 1), ("swiglu", 2, 300), ("swiglu", 1, 33),
                   ("geglu", 4, 40), ("geglu", 5, 129)]


@pytest.mark.parametrize("entry,codec,m", NONFINITE_CASES)
def test_non_finite_inputs_trip_exactly_their_rows_and_columns(torch, entry, codec, m):
    """A NaN or Inf activation makes its output row non-finite, an Inf scale
    makes its weight row's output column non-finite, and nothing leaks into
    other rows or columns, which stay within the tolerance of the oracle on
    clean data: the outputs' finite check (the pages' non-finite tripwire)
    fires exactly where the inputs are bad."""
    n, k, n_bad = 200, 512, 37
    seed = 6100 + codec + m
    x = synth.gen_x(m, k, seed)
    xb = x.copy()
    bad_rows = [m // 2] if m == 1 else [m // 2, m - 1]
    xb[bad_rows[0], 17] = np.float16(np.nan)
    if len(bad_rows) > 1:
        xb[bad_rows[1], 300] = np.float16(np.inf)
    gated = entry in ("swiglu", "geglu")
    mats = [synth.gen_weight(codec, n, k, seed, t) for t in ((synth.T_WG, synth.T_WU) if gated else (synth.T_W,))]
    bad = [_poison_scale(codec, mats[0], n, k, n_bad, 1)] + mats[1:]
    ws = [_weight(torch, codec, n, k, c) for c in bad]
    xd = _dev(torch, xb)
    if entry == "prefill":
        y = qg.qgemm_prefill(ws[0], xd)
    elif entry == "gemv":
        y = qg.qgemv_decode(ws[0], xd)
    elif entry == "swiglu":
        y = qg.qgemm_swiglu(ws[0], ws[1], xd)
    else:
        y = qg.qgemm_geglu(ws[0], ws[1], xd)
    y = y.cpu().numpy().astype(np.float64)
    want_bad = np.zeros((m, n), bool)
    want_bad[bad_rows, :] = True
    want_bad[:, n_bad] = True
    assert np.array_equal(~np.isfinite(y), want_bad)
    with pytest.raises(AssertionError, match="non-finite"):
        _err(y, np.ones_like(y))
    rows = np.setdiff1d(np.arange(m), bad_rows)
    cols = np.setdiff1d(np.arange(n), [n_bad])
    if len(rows):
        if gated:
            fn = oracle.swiglu_ref if entry == "swiglu" else oracle.geglu_ref
            ref = fn(codec, mats[0], mats[1], n, k, x[rows], rows_n=cols)
            assert _err_beyond_fp16_rounding(y[np.ix_(rows, cols)], ref) <= TOL
        else:
            ref = oracle.gemm_ref(codec, mats[0], n, k, x[rows], rows_n=cols)
            assert _err(y[np.ix_(rows, cols)], ref) <= TOL


def test_empty_batch_returns_empty_output_without_launch(torch):
    """X with no rows (an empty batch, with or without leading dims) gives an
    empty [..., N] result from every entry point; the C-ABI itself takes
    M >= 1 (QG_ERR_SHAPE for M = 0, checked on the host in test_lib_host)."""
    n, k = 64, 256
    w = _weight(torch, 1, n, k, synth.gen_weight(1, n, k, 31))
    wu = _weight(torch, 1, n, k, synth.gen_weight(1, n, k, 32))
    for shape in ((0, k), (3, 0, k)):
        x = torch.empty(shape, dtype=torch.float16, device="cuda")
        for y in (qg.qgemm_prefill(w, x), qg.qgemv_decode(w, x), qg.qgemm_swiglu(w, wu, x), qg.qgemm_geglu(w, wu, x)):
            assert tuple(y.shape) == shape[:-1] + (n,) and y.dtype == torch.float16 and y.is_cuda
    y = qg.qgemm_prefill_heads(w, torch.empty((0, k), dtype=torch.float16, device="cuda"), 32)
    assert tuple(y.shape) == (2, 0, 32)
    with pytest.raises(ValueError):
        qg.qgemm_prefill_heads(w, torch.empty((0, k), dtype=torch.float16, device="cuda"), 12)
    out = torch.empty((0, n), dtype=torch.float16, device="cuda")
    assert qg.qgemm_prefill(w, torch.empty((0, k), dtype=torch.float16, device="cuda"), out=out) is out
    kc, vc = synth.AttnWorkload("empty", 2, 1, 1, 64, 64, True, 5).kv()
    kv = qg.Q8KVCache.from_canonical(1, 64, 64, kc, vc)
    q = torch.empty((2, 0, 64), dtype=torch.float16, device="cuda")
    assert tuple(qg.qattn_prefill_q8kv(q, kv).shape) == (2, 0, 64)


@pytest.mark.parametrize("entry,m", [("prefill", 300), ("prefill", 40), ("gemv", 1), ("gemv", 3)])
def test_output_overflow_saturates_to_signed_infinity(torch, entry, m):
    """Y is fp16: an exact result beyond the largest binary16 (65504; with
    round-to-nearest-even everything from 65520 up) comes out as an infinity
    of its sign, every smaller one as a finite value within tolerance.  The
    rows are built far from the threshold on both sides: Q4_0 weights with
    d = 64 and codes 15 / 0 (w = +448 / -512) in alternate rows; X rows scaled
    so that some rows of Y reach about +-9e4 and the rest stay near 7e2."""
    n, k = 64, 256
    codes = np.where((np.arange(n) % 2 == 0)[:, None], 15, 0) * np.ones((n, k), np.int64)
    d = np.full((n, k // 32), 64.0, np.float16)
    canon = synth.encode_q4_0(codes.astype(np.uint8), d)
    w = _weight(torch, 1, n, k, canon)
    rng = np.random.default_rng(77)
    x = rng.uniform(0.5, 1.0, size=(m, k)).astype(np.float16)       # positive: the row sums do not cancel
    big = (np.arange(m) % 3 == 0)
    x[~big] *= np.float16(1.0 / 128.0)                               # |y| ~ 512 * 0.75 * 256 / 128 ~ 800
    ref = oracle.gemm_ref(1, canon, n, k, x)
    assert np.all(np.abs(ref[big]) > 1.2 * 65520) and np.all(np.abs(ref[~big]) < 65520 / 8)
    xd = torch.from_numpy(x).cuda()
    y = (qg.qgemm_prefill(w, xd) if entry == "prefill" else qg.qgemv_decode(w, xd)).cpu().numpy().astype(np.float64)
    assert np.all(np.isinf(y[big])) and np.array_equal(np.sign(y[big]), np.sign(ref[big]))
    small = ref[~big]
    if small.size:
        assert np.all(np.isfinite(y[~big]))
        assert float(np.max(np.abs(y[~big] - small)) / np.sqrt(np.mean(small ** 2))) <= TOL


def _big_q4_0(n, k, seed, tensor_id):
    """Q4_0 weights with d ~U(8, 16): |w| up to 128, so products with
    subnormal activations still sum to normal binary16 outputs (also through
    the gated product)."""
    rng = np.random.default_rng([seed, tensor_id])
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    return synth.encode_q4_0(codes, synth.fp16_uniform(rng, 8.0, 16.0, (n, k // 32)))


@pytest.mark.parametrize("entry,codec,m", [("prefill", 1, 200), ("prefill", 2, 40), ("gemv", 1, 1), ("gemv", 6, 4),
                                           ("swiglu", 1, 130)])
def test_subnormal_activations_are_not_flushed(torch, entry, codec, m):
    """X made entirely of binary16 subnormals (|x| < 2^-14): every product
    counts, so a kernel that flushed subnormal inputs to zero would return
    zeros against the oracle's nonzero result."""
    n, k = 96, 512
    gen = (lambda t: _big_q4_0(n, k, 880, t)) if codec == 1 else (lambda t: synth.gen_weight(codec, n, k, 880, t))
    canon, canon_u = gen(synth.T_W), gen(synth.T_WU)
    x = (synth.gen_x(m, k, 882).astype(np.float64) * 2.0 ** -18).astype(np.float16)
    assert np.all(np.abs(x.astype(np.float64)) < 2.0 ** -14) and np.count_nonzero(x) > 0.9 * x.size
    w, wu = _weight(torch, codec, n, k, canon), _weight(torch, codec, n, k, canon_u)
    xd = torch.from_numpy(x).cuda()
    if entry == "swiglu":
        y = qg.qgemm_swiglu(w, wu, xd)
        ref = oracle.swiglu(oracle.gemm_ref(codec, canon, n, k, x), oracle.gemm_ref(codec, canon_u, n, k, x))
    else:
        y = qg.qgemm_prefill(w, xd) if entry == "prefill" else qg.qgemv_decode(w, xd)
        ref = oracle.gemm_ref(codec, canon, n, k, x)
    y = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)) and np.count_nonzero(y) > 0.5 * y.size
    assert float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2))) <= TOL
