"""Pins for the oracle's hand-written binary16 conversions.

Library routine pin: numpy's float16 conversions are correctly rounded
(round to nearest, ties to even) in both directions, so the oracle must agree
with them bit for bit on every binary16 value, on every midpoint between
neighbours (the ties), one fp64 ulp either side of each midpoint, across the
subnormal range and at the overflow threshold.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_f16_to_f64_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signs of zeros survive
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _finite_f16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)].astype(np.float64)


def test_f64_to_f16_roundtrip_all_finite():
    v = _finite_f16_values()
    got = oracle.f64_to_f16_bits(v)
    assert np.array_equal(got, v.astype(np.float16).view(np.uint16))


def test_f64_to_f16_ties_and_neighbours():
    v = np.unique(_finite_f16_values())
    mids = (v[:-1] + v[1:]) / 2.0          # exact in fp64
    cand = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    got = oracle.f64_to_f16_bits(cand)
    want = cand.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f64_to_f16_random_and_edges():
    rng = np.random.default_rng(1234)
    mag = 10.0 ** rng.uniform(-12, 6, 200000)
    x = mag * np.where(rng.random(mag.size) < 0.5, -1.0, 1.0)
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e300, -65520.0,
                      2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 3 * 2.0 ** -26,
                      2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 5e-324, np.inf, -np.inf])
    x = np.concatenate([x, edges])
    got = oracle.f64_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f64_to_f16_nan():
    got = oracle.f64_to_f16_bits(np.array([np.nan]))
    assert np.isnan(got.view(np.float16)[0])
