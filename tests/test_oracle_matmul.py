"""Pins for the oracle's contraction and SwiGLU epilogue.

* Exact rational brute force on tiny inputs: the oracle's sequential fp64 sum
  must lie within the textbook error bound of recursive summation,
  |fl - exact| <= gamma_k * sum |x w| with gamma_k = k u / (1 - k u),
  u = 2^-53 -- a dropped term, a wrong sign, a shifted index or a transposed
  operand misses by orders of magnitude more.
* Library routine: BLAS fp64 matmul (numpy @) on the same decoded weights at
  the tiny Q4_0 workload's shape, to 1e-12 of rms.
* Row stride: X passed with ldx > K gives the same result as a packed copy.
* SwiGLU: out = SiLU(g) u against the independent identity
  sigma(g) = (1 + tanh(g / 2)) / 2, SiLU(0) = 0 and SiLU(g) - SiLU(-g) = g.
"""
import ctypes
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _exact_ref(x16, w):
    m, k = x16.shape
    n = w.shape[0]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            out[i, j] = sum(Fraction(float(x16[i, kk])) * Fraction(float(w[j, kk])) for kk in range(k))
    return out


@pytest.mark.parametrize("codec,k", [(1, 64), (2, 128), (3, 128), (4, 64), (5, 64), (6, 256), (7, 256)])
def test_matmul_exact_bruteforce(codec, k):
    m, n = 3, 5
    x = synth.gen_x(m, k, 17)
    canon = synth.gen_weight(codec, n, k, 18)
    w = oracle.decode(codec, canon, n, k)
    got = oracle.gemm_ref(codec, canon, n, k, x)
    exact = _exact_ref(x, w)
    u = 2.0 ** -53
    gamma = k * u / (1 - k * u)
    absw = np.abs(x.astype(np.float64)) @ np.abs(w).T
    for i in range(m):
        for j in range(n):
            err = abs(Fraction(got[i, j]) - exact[i, j])
            assert err <= Fraction(gamma * absw[i, j]) + Fraction(0), (i, j)
    # the bound is tight enough to catch a transposed or shifted operand
    assert got.shape == (m, n)


def test_matmul_matches_blas_tiny_workload():
    wl = synth.WORKLOADS["q4_0_tiny_16x256x256"]
    x = wl.x()
    (canon,) = wl.weights()
    ref = oracle.gemm_ref(wl.codec, canon, wl.n, wl.k, x)
    w = oracle.decode(wl.codec, canon, wl.n, wl.k)
    blas = x.astype(np.float64) @ w.T
    rms = np.sqrt(np.mean(blas ** 2))
    assert np.max(np.abs(ref - blas)) <= 1e-12 * rms


def test_matmul_row_subset_matches_full():
    codec, n, k = 3, 40, 256
    canon = synth.gen_weight(codec, n, k, 21)
    x = synth.gen_x(6, k, 22)
    full = oracle.gemm_ref(codec, canon, n, k, x)
    rows = np.array([0, 7, 39, 13])
    sub = oracle.gemm_ref(codec, canon, n, k, x, rows_n=rows)
    assert np.array_equal(sub, full[:, rows])
    canon2 = synth.gen_weight(2, n, k, 23)
    full2 = oracle.gemm_ref(2, canon2, n, k, x)
    sub2 = oracle.gemm_ref(2, canon2, n, k, x, rows_n=rows)
    assert np.array_equal(sub2, full2[:, rows])


def test_matmul_row_stride():
    m, n, k = 4, 6, 64
    x = synth.gen_x(m, k, 31)
    canon = synth.gen_weight(1, n, k, 32)
    w = oracle.decode(1, canon, n, k)
    padded = np.zeros((m, k + 24), dtype=np.float16)
    padded[:, :k] = x
    padded[:, k:] = np.float16(np.nan)     # must never be read
    out = np.empty((m, n), dtype=np.float64)
    xb = padded.view(np.uint16)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    oracle.lib().orc_matmul_xwt(p(xb), k + 24, p(w), m, n, k, p(out), 1)
    assert np.array_equal(out, oracle.matmul_xwt(x, w))


def test_matmul_thread_count_invariant():
    x = synth.gen_x(9, 128, 41)
    canon = synth.gen_weight(2, 33, 128, 42)
    w = oracle.decode(2, canon, 33, 128)
    assert np.array_equal(oracle.matmul_xwt(x, w, threads=1), oracle.matmul_xwt(x, w, threads=4))


def test_swiglu_identities():
    rng = np.random.default_rng(5)
    g = np.concatenate([rng.normal(0, 4, 10000), [0.0, -0.0, 30.0, -30.0, 700.0, -700.0, -800.0]])
    u = rng.normal(0, 2, g.size)
    got = oracle.swiglu(g, u)
    tanh_form = 0.5 * g * (1.0 + np.tanh(g / 2.0)) * u
    scale = np.maximum(np.abs(g * u), 1e-300)
    assert np.all(np.abs(got - tanh_form) <= 1e-14 * scale + 1e-300)
    assert oracle.swiglu(np.array([0.0]), np.array([3.0]))[0] == 0.0
    ones = np.ones_like(g)
    odd = oracle.swiglu(g, ones) - oracle.swiglu(-g, ones)
    assert np.allclose(odd, g, rtol=1e-13, atol=1e-13)
    assert np.all(np.isfinite(got))


def test_geglu_identities():
    """GELU in GeGLU is the tanh form.  Pins: GELU(0) = 0; the odd part of the
    tanh form is exactly the identity (0.5 g (1 + tanh t) + 0.5 g (1 - tanh t));
    GELU(g) -> g and -> 0 far out; and it stays within 1e-3 of the exact
    erf-based GELU everywhere (a dropped cubic term, a wrong sqrt(2/pi) or a
    sign slip all break that by an order of magnitude)."""
    from scipy.special import erf
    rng = np.random.default_rng(6)
    g = np.concatenate([rng.normal(0, 3, 20000), np.linspace(-8, 8, 4001), [0.0, -0.0, 30.0, -30.0]])
    ones = np.ones_like(g)
    got = oracle.geglu(g, ones)
    assert oracle.geglu(np.array([0.0]), np.array([5.0]))[0] == 0.0
    odd = got - oracle.geglu(-g, ones)
    assert np.allclose(odd, g, rtol=1e-13, atol=1e-13)
    exact = 0.5 * g * (1.0 + erf(g / np.sqrt(2.0)))
    assert np.max(np.abs(got - exact)) < 1e-3
    far = oracle.geglu(np.array([20.0, -20.0]), np.ones(2))
    assert abs(far[0] - 20.0) < 1e-12 and abs(far[1]) < 1e-12
    u = rng.normal(0, 2, g.size)
    assert np.allclose(oracle.geglu(g, u), got * u, rtol=1e-15, atol=0)



def test_non_finite_propagates_along_its_row_and_column():
    """IEEE rules the oracle inherits: a NaN or Inf activation makes its whole
    output row non-finite (x * 0 is NaN for x = Inf or NaN) and an Inf weight
    its whole output column; every other output stays finite."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64)).astype(np.float16)
    w = rng.standard_normal((5, 64))
    w[:, 10] = 0.0
    x[1, 10] = np.float16(np.nan)
    x[2, 20] = np.float16(np.inf)
    w[3, 40] = np.inf
    ref = oracle.matmul_xwt(x, w)
    bad = ~np.isfinite(ref)
    want = np.zeros((4, 5), bool)
    want[[1, 2], :] = True
    want[:, 3] = True
    assert np.array_equal(bad, want)
