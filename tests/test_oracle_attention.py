"""Pins for the attention oracle (oracle/attention.py).

Its Q8_0 decode is the weight decode pinned in test_oracle_decode.py.  Here
the attention itself is checked against closed forms that a dropped term, a
wrong mask direction, a missing scale, a wrong softmax axis, K and V swapped or
a wrong grouped-query mapping would each break:
* a single visible key returns its V row exactly (one key; the first query of
  a causal prefill);
* zero queries weight the visible keys uniformly: the output is the plain mean
  of the visible V rows;
* two keys: the weights are sigma(a - b) and sigma(b - a), with sigma taken
  from the independent identity sigma(t) = (1 + tanh(t / 2)) / 2;
* without the mask, a joint permutation of the K and V rows changes nothing;
* grouped-query heads read KV head h // (H / H_kv).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.attention import q8kv_attention_ref


def _q8(rows, d, seed):
    return synth.gen_q8_0(rows, d, seed, d_range=(0.01, 0.03))


def _kv(canon, rows, d):
    return oracle.decode(oracle.Q8_0, canon, rows, d)


def test_single_key_returns_its_value_row():
    d = 64
    q = synth.gen_x(1, d, 1).reshape(1, 1, d)
    kc, vc = _q8(1, d, 2), _q8(1, d, 3)
    out = q8kv_attention_ref(q, kc, vc, 1, 1, causal=True, scale=0.125)
    assert np.array_equal(out[0, 0], _kv(vc, 1, d)[0])


def test_causal_first_query_sees_only_the_first_key():
    h, m, d = 2, 5, 64
    q = synth.gen_x(h * m, d, 4).reshape(h, m, d)
    kc, vc = _q8(m, d, 5), _q8(m, d, 6)
    out = q8kv_attention_ref(q, kc, vc, 1, m, causal=True, scale=0.125)
    v = _kv(vc, m, d)
    assert np.array_equal(out[0, 0], v[0]) and np.array_equal(out[1, 0], v[0])


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_average_the_visible_values(causal):
    h, m, s, d = 2, 6, 9, 32
    q = np.zeros((h, m, d), np.float16)
    kc, vc = _q8(s, d, 7), _q8(s, d, 8)
    out = q8kv_attention_ref(q, kc, vc, 1, s, causal=causal, scale=0.3)
    v = _kv(vc, s, d)
    for i in range(m):
        visible = (s - m) + i + 1 if causal else s
        assert np.allclose(out[0, i], v[:visible].mean(axis=0), rtol=0, atol=1e-14)


def test_two_keys_closed_form():
    d = 32
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, d)).astype(np.float16)
    kc, vc = _q8(2, d, 10), _q8(2, d, 11)
    k, v = _kv(kc, 2, d), _kv(vc, 2, d)
    scale = 0.7
    qf = q.astype(np.float64)[0, 0]
    a, b = scale * float(qf @ k[0]), scale * float(qf @ k[1])
    sig = lambda t: (1.0 + np.tanh(t / 2.0)) / 2.0
    want = sig(a - b) * v[0] + sig(b - a) * v[1]
    out = q8kv_attention_ref(q, kc, vc, 1, 2, causal=False, scale=scale)
    assert np.allclose(out[0, 0], want, rtol=1e-13, atol=1e-15)


def test_key_permutation_invariance_without_mask():
    h, m, s, d = 1, 4, 16, 64
    q = synth.gen_x(m, d, 12).reshape(h, m, d)
    kc, vc = _q8(s, d, 13), _q8(s, d, 14)
    perm = np.random.default_rng(15).permutation(s)
    kp = kc.reshape(s, -1)[perm].reshape(-1)
    vp = vc.reshape(s, -1)[perm].reshape(-1)
    a = q8kv_attention_ref(q, kc, vc, 1, s, causal=False, scale=0.125)
    b = q8kv_attention_ref(q, kp, vp, 1, s, causal=False, scale=0.125)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_grouped_query_heads_use_their_kv_head():
    heads, kv_heads, m, d = 4, 2, 3, 64
    q = synth.gen_x(heads * m, d, 16).reshape(heads, m, d)
    kc, vc = _q8(kv_heads * m, d, 17), _q8(kv_heads * m, d, 18)
    out = q8kv_attention_ref(q, kc, vc, kv_heads, m, causal=True, scale=0.125)
    row_bytes = (d // 32) * 34
    for h in range(heads):
        g = h // 2
        ks = kc[g * m * row_bytes:(g + 1) * m * row_bytes]
        vs = vc[g * m * row_bytes:(g + 1) * m * row_bytes]
        single = q8kv_attention_ref(q[h:h + 1], ks, vs, 1, m, causal=True, scale=0.125)
        assert np.array_equal(out[h], single[0])


def test_row_subset_matches_full():
    heads, m, s, d = 2, 7, 12, 64
    q = synth.gen_x(heads * m, d, 19).reshape(heads, m, d)
    kc, vc = _q8(s, d, 20), _q8(s, d, 21)
    full = q8kv_attention_ref(q, kc, vc, 1, s, causal=True, scale=0.125)
    rows = np.array([0, 3, 6])
    sub = q8kv_attention_ref(q, kc, vc, 1, s, causal=True, scale=0.125, rows=rows)
    assert np.array_equal(full[:, rows], sub)


def test_fp16_kv_option_uses_the_rounded_cache():
    """kv_f16 reads every K and V element as its correctly rounded binary16:
    the single visible key returns exactly numpy's fp16 rounding of the exact
    V row (which differs from the exact row somewhere for these scales), the
    zero-query average is the mean of the rounded rows, and on random data the
    result stays within fp16 rounding of the exact-cache result."""
    d = 64
    q = synth.gen_x(1, d, 11).reshape(1, 1, d)
    kc, vc = _q8(1, d, 12), _q8(1, d, 13)
    exact = _kv(vc, 1, d)[0]
    out = q8kv_attention_ref(q, kc, vc, 1, 1, causal=True, scale=0.125, kv_f16=True)
    assert np.array_equal(out[0, 0], exact.astype(np.float16).astype(np.float64))
    assert not np.array_equal(out[0, 0], exact)
    h, m, s = 1, 3, 7
    kc, vc = _q8(s, d, 14), _q8(s, d, 15)
    z = q8kv_attention_ref(np.zeros((h, m, d), np.float16), kc, vc, 1, s, causal=False, scale=0.3, kv_f16=True)
    v16 = _kv(vc, s, d).astype(np.float16).astype(np.float64)
    assert np.allclose(z[0, 0], v16.mean(axis=0), rtol=0, atol=1e-14)
    q = synth.gen_x(2 * 40, d, 16).reshape(2, 40, d)
    kc, vc = _q8(40, d, 17), _q8(40, d, 18)
    a = q8kv_attention_ref(q, kc, vc, 1, 40, causal=True, scale=0.125)
    b = q8kv_attention_ref(q, kc, vc, 1, 40, causal=True, scale=0.125, kv_f16=True)
    assert 0 < np.max(np.abs(a - b)) <= 4 * 2.0 ** -11 * np.max(np.abs(a))
