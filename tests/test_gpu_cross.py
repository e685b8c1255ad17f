"""Boundary cross-product: every codec x every GEMM / GEMV entry point x the
token counts the dispatch tells apart, element by element against the oracle.

The releases page (v0.2.3, bit-exact parity suite; v0.3.0, verification and
test coverage) checks every codec at each boundary token count; here those are
M in {1, 2, 3, 4} (the weight-streaming kernel's row counts), 33 and 64 (one
64-row split-k tile), 127 and 128 (two), 129 and 512 (the 128-row prefill
tiles), on a ragged N of 200 (six full 32-row groups and a partial one) and
K = 512 (eight k-steps: two per k-slice of the split-k tiles; four Q2_0
blocks, two Q4_K / ternary super-blocks).  Which kernel instantiation each
case reaches is reported by qg_kernel_for; tests/test_dispatch_coverage.py
shows on the host that these cases, together with the other GPU tests, reach
every instantiation the C-ABI can launch.

Q8_0 codes are drawn over the whole byte range, -128 included (the oracle pins
-128 as -128 d).  Gated outputs report the raw max|err|/rms beside the error
beyond the fp16 output's own half-ulp rounding that the bar applies to.
"""
import numpy as np
import pytest

import oracle
import synth
import quantized_prefill_gemm_codec_amd as qg

pytestmark = pytest.mark.gpu

TOL = 1e-2
CODECS = [1, 2, 3, 4, 5, 6, 7, 8]
ENTRIES = ["prefill", "heads", "swiglu", "geglu", "gemv"]
MS = [1, 2, 3, 4, 33, 64, 127, 128, 129, 512]
N, K, HEAD_DIM = 200, 512, 40


def cross_cases():
    return [(c, e, m) for c in CODECS for e in ENTRIES for m in MS]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no HIP device")
    return t


def q8_0_full_range(n, k, seed, tensor_id):
    """Q8_0 weights with codes ~U{-128..127}; the first code of every row is
    -128, so each row group and k-slice of the kernels meets it."""
    rng = np.random.default_rng([seed, tensor_id])
    codes = rng.integers(-128, 128, size=(n, k), dtype=np.int16).astype(np.int8)
    codes[:, 0] = -128
    codes[::3, k // 2 + 5] = -128
    d = synth.fp16_uniform(rng, 0.0005, 0.0015, (n, k // 32))
    return synth.encode_q8_0(codes, d)


def _canon(codec, tensor_id):
    seed = 7700 + codec
    if codec == 4:
        return q8_0_full_range(N, K, seed, tensor_id)
    return synth.gen_weight(codec, N, K, seed, tensor_id)


_DATA = {}


def _data(torch, codec):
    """Weights, X [512, K] and the oracle's fp64 products, once per codec; the
    case with M rows uses the first M rows of X (and of the products)."""
    if codec not in _DATA:
        x = synth.gen_x(max(MS), K, 7800 + codec)
        mats = {t: _canon(codec, t) for t in (synth.T_W, synth.T_WG, synth.T_WU)}
        refs = {t: oracle.gemm_ref(codec, c, N, K, x) for t, c in mats.items()}
        ws = {t: qg.QWeight.from_canonical(codec, N, K, c, device="cuda") for t, c in mats.items()}
        _DATA[codec] = (x, ws, refs)
    return _DATA[codec]


def _rel(y, ref):
    return float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)))


def _beyond_rounding(y, ref):
    return float(np.max(np.maximum(np.abs(y - ref) - 2.0 ** -11 * np.abs(ref), 0.0)) / np.sqrt(np.mean(ref ** 2)))


@pytest.mark.parametrize("codec,entry,m", cross_cases())
def test_cross_product(torch, record_property, codec, entry, m):
    x, ws, refs = _data(torch, codec)
    kernel = qg.qg_kernel_for(entry, codec, m, N, K) if not (entry == "gemv" and m > 64) else None
    record_property("kernel", kernel)
    xd = torch.from_numpy(np.ascontiguousarray(x[:m])).cuda()
    if entry == "gemv" and m > 64:
        with pytest.raises(qg.QGError) as e:
            qg.qgemv_decode(ws[synth.T_W], xd)
        assert e.value.status == -3          # QG_ERR_SHAPE: the GEMV takes at most 64 rows
        return
    if entry == "prefill":
        y = qg.qgemm_prefill(ws[synth.T_W], xd)
    elif entry == "heads":
        y = qg.qgemm_prefill_heads(ws[synth.T_W], xd, HEAD_DIM).permute(1, 0, 2).reshape(m, N)
    elif entry == "gemv":
        y = qg.qgemv_decode(ws[synth.T_W], xd)
    elif entry == "swiglu":
        y = qg.qgemm_swiglu(ws[synth.T_WG], ws[synth.T_WU], xd)
    else:
        y = qg.qgemm_geglu(ws[synth.T_WG], ws[synth.T_WU], xd)
    y = y.cpu().numpy().astype(np.float64)
    assert y.shape == (m, N)
    assert np.all(np.isfinite(y)), f"non-finite output from {kernel}"
    if entry in ("swiglu", "geglu"):
        fn = oracle.swiglu if entry == "swiglu" else oracle.geglu
        ref = fn(refs[synth.T_WG][:m], refs[synth.T_WU][:m])
        raw, beyond = _rel(y, ref), _beyond_rounding(y, ref)
        record_property("err_report", f"{entry} codec={codec} m={m} {kernel}: raw max|err|/rms={raw:.4g}, "
                                      f"beyond fp16 output rounding={beyond:.4g}")
        assert beyond <= TOL, (kernel, raw, beyond)
    else:
        err = _rel(y, refs[synth.T_W][:m])
        assert err <= TOL, (kernel, err)
