"""GPU parity at the edges of the shape range, through the C-ABI.

* Degenerate shapes: a single output column (N = 1), K equal to one codec
  block, one query row through the prefill entry point, very tall X against a
  handful of weight rows.
* Large sizes: a K of 2^18 weights (4096 k-steps through the 32-bit offset
  arithmetic), a 537 MB weight plane streamed by the decode and the prefill
  kernels, and attention over a 32767-position cache.  These are checked on
  rows and columns sampled the way the full-workload tests sample them; the
  oracle computes exactly those.
Tolerance as everywhere: max |err| / rms(ref) <= 1e-2 of the fp64 oracle.
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


def _err(y, ref):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    return float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)))


def _sample(rng, size, count):
    if size <= count:
        return np.arange(size)
    s = rng.choice(np.arange(1, size - 1), count - 2, replace=False)
    return np.sort(np.concatenate([[0, size - 1], s]))


DEGENERATE = [
    # codec, m, n, k
    (1, 1, 1, 32), (1, 3000, 1, 32), (1, 130, 1, 64), (2, 5000, 7, 64), (3, 64, 33, 128), (4, 200, 1, 32),
    (5, 7, 3, 32), (6, 1, 1, 256), (6, 129, 2, 256), (7, 2, 1, 256), (7, 300, 5, 256),
]


@pytest.mark.parametrize("codec,m,n,k", DEGENERATE)
def test_degenerate_shapes(torch, codec, m, n, k):
    seed = 9000 + codec + m + n + k
    canon = synth.gen_weight(codec, n, k, seed)
    x = synth.gen_x(m, k, seed)
    w = qg.QWeight.from_canonical(codec, n, k, canon, device="cuda")
    y = qg.qgemm_prefill(w, torch.from_numpy(x).cuda()).cpu().numpy()
    assert y.shape == (m, n)
    assert _err(y, oracle.gemm_ref(codec, canon, n, k, x)) <= TOL


def test_long_k(torch):
    """K = 2^18: 4096 k-steps, X rows of 512 KiB, ragged M."""
    codec, m, n, k = 1, 257, 256, 1 << 18
    canon = synth.gen_weight(codec, n, k, 9101)
    x = synth.gen_x(m, k, 9101)
    w = qg.QWeight.from_canonical(codec, n, k, canon, device="cuda")
    y = qg.qgemm_prefill(w, torch.from_numpy(x).cuda()).cpu().numpy()
    rng = np.random.default_rng(9101)
    rows_m, rows_n = _sample(rng, m, 8), _sample(rng, n, 64)
    ref = oracle.gemm_ref(codec, canon, n, k, x[rows_m], rows_n=rows_n)
    assert _err(y[np.ix_(rows_m, rows_n)], ref) <= TOL


@pytest.fixture(scope="module")
def big_weight(torch):
    """A [131072, 8192] Q4_0 weight: 537 MB of codes on the device."""
    codec, n, k = 1, 131072, 8192
    canon = synth.gen_weight(codec, n, k, 9102)
    w = qg.QWeight.from_canonical(codec, n, k, canon, device="cuda")
    yield codec, n, k, canon, w
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [1, 300])
def test_half_gigabyte_weight(torch, big_weight, m):
    """The 537 MB weight through the decode GEMV (m = 1) and the prefill GEMM (m = 300)."""
    codec, n, k, canon, w = big_weight
    x = synth.gen_x(m, k, 9103)
    y = qg.qgemm_prefill(w, torch.from_numpy(x).cuda()).cpu().numpy()
    rng = np.random.default_rng(9102 + m)
    rows_m, rows_n = _sample(rng, m, 6), _sample(rng, n, 256)
    ref = oracle.gemm_ref(codec, canon, n, k, x[rows_m], rows_n=rows_n)
    assert _err(y[np.ix_(rows_m, rows_n)], ref) <= TOL


def test_attention_long_context(torch):
    """255 queries at the end of a 32767-position Q8_0 cache (both ragged)."""
    heads, kv_heads, m, s, d = 2, 1, 255, 32767, 128
    wl = synth.AttnWorkload("long", heads, kv_heads, m, s, d, True, 9104)
    q = wl.q()
    kc, vc = wl.kv()
    cache = qg.Q8KVCache.from_canonical(kv_heads, s, d, kc, vc)
    out = qg.qattn_prefill_q8kv(torch.from_numpy(q).cuda(), cache, causal=True, scale=1.0 / np.sqrt(d))
    got = out.cpu().numpy().astype(np.float64)
    rows = _sample(np.random.default_rng(9104), m, 10)
    ref = q8kv_attention_ref(q, kc, vc, kv_heads, s, True, np.float32(1.0 / np.sqrt(d)).item(), rows=rows)
    assert _err(got[:, rows], ref) <= TOL


@pytest.mark.parametrize("nbytes", [16, 1008, 1 << 20, 33030144 + 16 * 37])
def test_stream_read_checksum(torch, nbytes):
    """The calibration read touches every byte once: its XOR checksum equals
    numpy's over the same words, ragged shares and tails included."""
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    want = int(np.bitwise_xor.reduce(words))
    src = torch.from_numpy(words.view(np.int32)).cuda()
    assert qg.qg_stream_read(src) == want
    slots = torch.zeros(qg.QG_STREAM_READ_SLOTS, dtype=torch.int32, device="cuda")
    qg.qg_stream_read(src, out=slots)
    assert int(np.bitwise_xor.reduce(slots.cpu().numpy().view(np.uint32))) == want
    qg.qg_stream_read(src, out=slots)
    assert not slots.cpu().numpy().any()      # every slot XORed with the same partial twice

