"""GPU parity of the Q8_0-KV attention kernel against the fp64 oracle
(oracle/attention.py), through the C-ABI entry point qattn_prefill_q8kv.

Tolerance: max |O - ref| / rms(ref) <= 1e-2, as for the GEMM outputs.  The
kernel's own rounding (K, V rounded once to fp16, P rounded to fp16 for the
second product, fp32 sums, fp16 output) is about 1e-3 of rms.
"""
import numpy as np
import pytest

import oracle
import synth
import quantized_prefill_gemm_codec_amd as qg
from oracle.attention import q8kv_attention_ref

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no HIP device")
    return t


def _run(torch, heads, kv_heads, m, s, d, causal, seed, rows=None, scale=None):
    wl = synth.AttnWorkload("t", heads, kv_heads, m, s, d, causal, seed)
    q = wl.q()
    kc, vc = wl.kv()
    cache = qg.Q8KVCache.from_canonical(kv_heads, s, d, kc, vc)
    sc = scale if scale is not None else 1.0 / np.sqrt(d)
    out = qg.qattn_prefill_q8kv(torch.from_numpy(q).cuda(), cache, causal=causal, scale=sc)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = q8kv_attention_ref(q, kc, vc, kv_heads, s, causal, np.float32(sc).item(), rows=rows)
    if rows is not None:
        got = got[:, rows]
    return got, ref, out


def _err(got, ref):
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


SHAPES = [
    # heads, kv_heads, m, s, d, causal
    (1, 1, 1, 1, 64, True), (2, 1, 5, 5, 64, True), (4, 2, 64, 64, 128, True), (4, 4, 100, 100, 64, True),
    (8, 2, 130, 200, 128, True), (2, 2, 77, 300, 64, False), (3, 1, 129, 129, 128, False),
    (2, 1, 1, 500, 128, True), (4, 1, 256, 256, 128, True), (2, 2, 200, 520, 64, True), (1, 1, 63, 65, 128, False),
]


@pytest.mark.parametrize("heads,kv_heads,m,s,d,causal", SHAPES)
def test_attention_parity(torch, heads, kv_heads, m, s, d, causal):
    got, ref, _ = _run(torch, heads, kv_heads, m, s, d, causal, 7000 + heads + m + s + d)
    assert _err(got, ref) <= TOL


def test_attention_first_query_is_first_value_row(torch):
    """Causal, m = s: query 0 sees key 0 only, so O[h, 0] is V[g, 0] rounded to fp16 (twice: K/V dequant and output)."""
    heads, kv_heads, m, d = 4, 2, 70, 128
    got, _, _ = _run(torch, heads, kv_heads, m, m, d, True, 7101)
    wl = synth.AttnWorkload("t", heads, kv_heads, m, m, d, True, 7101)
    _, vc = wl.kv()
    v = oracle.dequant_f16_bits(oracle.Q8_0, vc, kv_heads * m, d).view(np.float16).astype(np.float64)
    for h in range(heads):
        assert np.array_equal(got[h, 0], v[(h // 2) * m])


def test_attention_is_deterministic(torch):
    _, _, a = _run(torch, 4, 2, 150, 150, 64, True, 7102)
    _, _, b = _run(torch, 4, 2, 150, 150, 64, True, 7102)
    assert np.array_equal(a.cpu().numpy().view(np.uint16), b.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("name", list(synth.ATTN_WORKLOADS))
def test_attention_full_workload_sampled(torch, name):
    wl = synth.ATTN_WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    rows = np.sort(np.concatenate([[0, wl.m - 1], rng.choice(np.arange(1, wl.m - 1), 30, replace=False)]))
    got, ref, _ = _run(torch, wl.heads, wl.kv_heads, wl.m, wl.s, wl.head_dim, wl.causal, wl.seed, rows=rows)
    assert _err(got, ref) <= TOL


def _run_inputs(torch, q, kc, vc, kv_heads, s, d, causal, scale, kv_f16=False):
    cache = qg.Q8KVCache.from_canonical(kv_heads, s, d, kc, vc)
    out = qg.qattn_prefill_q8kv(torch.from_numpy(q).cuda(), cache, causal=causal, scale=scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    return got, q8kv_attention_ref(q, kc, vc, kv_heads, s, causal, np.float32(scale).item(), kv_f16=kv_f16)


@pytest.mark.parametrize("d,order", [(128, "rising"), (64, "rising"), (128, "falling"), (64, "peaked")])
def test_attention_running_maximum_paths(torch, d, order):
    """Scores that rise along the keys move the rows' running maximum every few
    64-key tiles (the accumulators are rescaled each time), and with an 8x
    scale ("peaked", a nearly one-hot softmax) in every tile; falling scores
    never move it after the first tile.  The reference reads the cache at the
    kernel's operand precision (every K and V element rounded once to fp16):
    with scores this large the rounding of K alone moves a nearly one-hot
    softmax by more than 1e-2 of rms against the exact cache, while this test
    is about the online softmax's arithmetic."""
    heads, kv_heads, m, s = 4, 2, 96, 640
    wl = synth.AttnWorkload("t", heads, kv_heads, m, s, d, True, 7300 + d)
    q = np.abs(wl.q()).astype(np.float16)                 # positive queries
    kc, vc = wl.kv()
    blocks = d // 32
    k8 = kc.reshape(kv_heads * s, blocks, 34).copy()
    codes = np.abs(k8[:, :, 2:].view(np.int8).astype(np.int16))    # positive keys: score ~ (d-scale) * key position
    pos = np.tile(np.arange(s), kv_heads)
    ramp = (pos + 1) / s if order != "falling" else (s - pos) / s
    k8[:, :, 2:] = np.clip(codes * ramp[:, None, None], 0, 127).astype(np.int8).view(np.uint8)
    kc = k8.reshape(-1)
    scale = (8.0 if order == "peaked" else 1.0) / np.sqrt(d)
    got, ref = _run_inputs(torch, q, kc, vc, kv_heads, s, d, True, scale, kv_f16=True)
    assert _err(got, ref) <= TOL


def test_attention_code_minus_128(torch):
    """K and V codes of -128 (byte 0x80, the one code outside +-127) decode as
    -128 d through the kernel's stored q + 128, as the oracle reads them."""
    heads, kv_heads, m, s, d = 2, 1, 80, 80, 128
    wl = synth.AttnWorkload("t", heads, kv_heads, m, s, d, True, 7400)
    q = wl.q()
    kc, vc = wl.kv()
    kb = kc.reshape(kv_heads * s, d // 32, 34).copy()
    vb = vc.reshape(kv_heads * s, d // 32, 34).copy()
    kb[::3, :, 2::5] = 0x80
    vb[1::2, :, 3::4] = 0x80
    got, ref = _run_inputs(torch, q, kb.reshape(-1), vb.reshape(-1), kv_heads, s, d, True, 1.0 / np.sqrt(d))
    assert _err(got, ref) <= TOL
