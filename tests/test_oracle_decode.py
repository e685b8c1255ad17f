"""Pins for the oracle's exact codec decode.

* Hand-worked fixtures (tests/golden/*.txt): byte strings whose weights follow
  from the formulas on the pages by hand -- Q2_0 w = (q - 1) d with q = 3 -> +2d
  in 34-byte, 128-weight blocks; Q4_0 w = (q - 8) d in 18-byte, 32-weight
  blocks; MLX w = q s + b per 64-weight group; Q8_0 w = q d with q a signed
  byte (GGUF block_q8_0, a reading); Q4_K w = d sc q - dmin m over 256-weight,
  144-byte super-blocks with 6-bit sub-block fields (public GGUF layout, a
  reading).  They fix the offsets, signs, nibble / bit order, block strides and
  row strides.
* Ternary 1.58-bit (base-3 digits, five per byte, a reading) is further
  pinned by an exhaustive sweep of all 243 valid byte values in every byte
  position against repeated division by 3, and by rejection of invalid bytes.
* Q4_K is further pinned by a special case that reduces to the fixture-pinned
  Q4_0 decode, an exhaustive sweep of its 6-bit fields and exact rational
  arithmetic at extreme scale ratios.
* Geometry printed on the pages: Q2_0 is 2.125 bits per weight.
* Closed forms: MLX q = 0 gives the bias bit for bit; the fp16 image of each
  weight equals numpy's correctly rounded conversion of the exact value.
* The seeded generator's encoders agree with the oracle's reading of the
  canonical bytes (so GPU parity inputs mean what the fixtures say).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from golden_io import all_cases

CASES = all_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_decode(case):
    canon = np.array(case["bytes"], dtype=np.uint8)
    assert canon.size == synth.canonical_bytes(case["codec"], case["n"], case["k"])
    w = oracle.decode(case["codec"], canon, case["n"], case["k"])
    want = np.array(case["expect"], dtype=np.float64).reshape(case["n"], case["k"])
    assert np.array_equal(w, want)


def test_q2_0_bits_per_weight_printed_on_page():
    weights, nbytes = oracle.block_geometry(oracle.Q2_0)
    assert (weights, nbytes) == (128, 34)
    assert nbytes * 8 / weights == 2.125


def test_q4_0_geometry():
    assert oracle.block_geometry(oracle.Q4_0) == (32, 18)


def test_mlx4_g32_is_the_pages_20_byte_block():
    # comparison page, section 4: block_mlx_4bit is 20 bytes (20 mod 16 = 4)
    weights, nbytes = oracle.block_geometry(oracle.MLX4_G32)
    assert (weights, nbytes) == (32, 20) and nbytes % 16 == 4


def test_q8_0_geometry():
    weights, nbytes = oracle.block_geometry(oracle.Q8_0)
    assert (weights, nbytes) == (32, 34)
    assert nbytes * 8 / weights == 8.5


def test_q4_k_geometry():
    weights, nbytes = oracle.block_geometry(oracle.Q4_K)
    assert (weights, nbytes) == (256, 144)
    assert nbytes * 8 / weights == 4.5


def test_q4_k_with_unit_scales_is_q4_0():
    # sc = 1, m = 8 and dmin = d make every Q4_K weight d q - 8 d, the Q4_0
    # formula with that d in each of the super-block's eight 32-weight blocks
    rng = np.random.default_rng(21)
    n, k = 3, 512
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    d = rng.uniform(0.005, 0.02, (n, k // 256)).astype(np.float16)
    q4k = synth.encode_q4_k(codes, np.ones((n, k // 32), np.uint8), np.full((n, k // 32), 8, np.uint8), d, d)
    q40 = synth.encode_q4_0(codes, np.repeat(d, 8, axis=1))
    assert np.array_equal(oracle.decode(oracle.Q4_K, q4k, n, k), oracle.decode(oracle.Q4_0, q40, n, k))


def test_q4_k_six_bit_fields_exhaustive():
    # every value 0..63 in every sub-block position, for scales (d = 1, dmin = 0,
    # q = 1: w = sc) and for mins (d = 0, dmin = -1: w = m)
    n, k = 64, 256
    vals = (np.arange(n)[:, None] + 7 * np.arange(8)[None, :]) % 64
    ones = np.ones((n, k), np.uint8)
    zeros8 = np.zeros((n, 8), np.uint8)
    unit, zero, neg = (np.full((n, 1), v, np.float16) for v in (1.0, 0.0, -1.0))
    w_sc = oracle.decode(oracle.Q4_K, synth.encode_q4_k(ones, vals, zeros8, unit, zero), n, k)
    w_m = oracle.decode(oracle.Q4_K, synth.encode_q4_k(ones, zeros8, vals, zero, neg), n, k)
    assert np.array_equal(w_sc, np.repeat(vals, 32, axis=1).astype(np.float64))
    assert np.array_equal(w_m, np.repeat(vals, 32, axis=1).astype(np.float64))


def test_q4_k_decode_exact_at_extreme_ratios():
    # d and dmin from the largest normal to the smallest subnormal binary16:
    # the fp64 decode must equal the exact rational d sc q - dmin m
    pats = np.array([0x7BFF, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x3555, 0xFBFF, 0x8001, 0x1234, 0x6A5A],
                    dtype=np.uint16)
    pairs = [(a, b) for a in pats for b in pats]
    n, k = len(pairs), 256
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    sc = rng.integers(0, 64, (n, 8)).astype(np.uint8)
    mn = rng.integers(0, 64, (n, 8)).astype(np.uint8)
    sc[:, 0] = 63
    mn[:, 0] = 63
    codes[:, :32] = 15
    d = np.array([a for a, _ in pairs], np.uint16).view(np.float16).reshape(n, 1)
    dmin = np.array([b for _, b in pairs], np.uint16).view(np.float16).reshape(n, 1)
    w = oracle.decode(oracle.Q4_K, synth.encode_q4_k(codes, sc, mn, d, dmin), n, k)
    for r in range(n):
        fd, fm = Fraction(float(d[r, 0])), Fraction(float(dmin[r, 0]))
        for kk in range(0, k, 7):
            j = kk // 32
            exact = fd * int(sc[r, j]) * int(codes[r, kk]) - fm * int(mn[r, j])
            assert Fraction(w[r, kk]) == exact


def test_ternary_geometry():
    weights, nbytes = oracle.block_geometry(oracle.TERNARY)
    assert (weights, nbytes) == (256, 54)
    assert nbytes * 8 / weights == 1.6875          # log2(3) = 1.585 for the digits alone


def test_ternary_all_byte_values_exhaustive():
    # byte values 0..242 spread over the 51 five-digit bytes of 5 rows; weight
    # 255 (digit 0 of byte 53) cycles through 0..2
    n, k = 5, 256
    vals = np.arange(n * 51) % 243
    canon = np.zeros((n, 54), np.uint8)
    canon[:, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)   # d = 1
    canon[:, 2:53] = vals.reshape(n, 51)
    canon[:, 53] = np.arange(n) % 3
    w = oracle.decode(oracle.TERNARY, canon.reshape(-1), n, k)
    want = np.empty((n, k))
    for r in range(n):
        for j in range(51):
            v = int(canon[r, 2 + j])
            for i in range(5):
                v, t = divmod(v, 3)
                want[r, 5 * j + i] = t - 1
        want[r, 255] = int(canon[r, 53]) - 1
    assert np.array_equal(w, want)


@pytest.mark.parametrize("pos,val", [(2, 243), (30, 255), (53, 3)])
def test_ternary_rejects_invalid_bytes(pos, val):
    canon = np.zeros(54, np.uint8)
    canon[pos] = val
    with pytest.raises(ValueError):
        oracle.decode(oracle.TERNARY, canon, 1, 256)


def test_decode_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.decode(oracle.Q4_0, np.zeros(18, np.uint8), 1, 48)
    with pytest.raises(ValueError):
        oracle.decode(9, np.zeros(18, np.uint8), 1, 32)


def test_mlx_zero_code_returns_bias_bits():
    rng = np.random.default_rng(7)
    n, k = 8, 256
    codes = np.zeros((n, k), np.uint8)
    s = rng.uniform(0.002, 0.01, (n, k // 64)).astype(np.float16)
    b = (0.02 * rng.standard_normal((n, k // 64))).astype(np.float16)
    b[0, 0] = np.float16(2.0 ** -20)     # subnormal bias survives
    canon = synth.encode_mlx4(codes, s, b)
    bits = oracle.dequant_f16_bits(oracle.MLX4_G64, canon, n, k)
    want = np.repeat(b.view(np.uint16), 64, axis=1)
    assert np.array_equal(bits, want)


def _random_canon(codec, n, k, seed):
    return synth.gen_weight(codec, n, k, seed)


@pytest.mark.parametrize("codec", [1, 2, 3, 4, 5, 6, 7])
def test_dequant_f16_matches_numpy_rounding(codec):
    n, k = 16, 512
    canon = _random_canon(codec, n, k, 99)
    w = oracle.decode(codec, canon, n, k)
    bits = oracle.dequant_f16_bits(codec, canon, n, k)
    assert np.array_equal(bits, w.astype(np.float16).view(np.uint16))


def test_generator_q4_0_encoding_matches_decode():
    rng = np.random.default_rng(3)
    n, k = 5, 96
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    d = rng.uniform(0.005, 0.02, (n, k // 32)).astype(np.float16)
    w = oracle.decode(1, synth.encode_q4_0(codes, d), n, k)
    want = (codes.astype(np.float64) - 8) * np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.array_equal(w, want)


def test_generator_mlx4_encoding_matches_decode():
    rng = np.random.default_rng(4)
    n, k = 3, 192
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    s = rng.uniform(0.002, 0.01, (n, k // 64)).astype(np.float16)
    b = (0.02 * rng.standard_normal((n, k // 64))).astype(np.float16)
    w = oracle.decode(2, synth.encode_mlx4(codes, s, b), n, k)
    want = codes * np.repeat(s.astype(np.float64), 64, axis=1) + np.repeat(b.astype(np.float64), 64, axis=1)
    assert np.array_equal(w, want)


def test_generator_mlx4_g32_encoding_matches_decode():
    rng = np.random.default_rng(8)
    n, k = 3, 160
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    s = rng.uniform(0.002, 0.01, (n, k // 32)).astype(np.float16)
    b = (0.02 * rng.standard_normal((n, k // 32))).astype(np.float16)
    w = oracle.decode(5, synth.encode_mlx4(codes, s, b), n, k)
    want = codes * np.repeat(s.astype(np.float64), 32, axis=1) + np.repeat(b.astype(np.float64), 32, axis=1)
    assert np.array_equal(w, want)


def test_generator_q2_0_encoding_matches_decode():
    rng = np.random.default_rng(5)
    n, k = 4, 256
    codes = rng.integers(0, 4, (n, k)).astype(np.uint8)
    d = rng.uniform(0.01, 0.05, (n, k // 128)).astype(np.float16)
    w = oracle.decode(3, synth.encode_q2_0(codes, d), n, k)
    want = (codes.astype(np.float64) - 1) * np.repeat(d.astype(np.float64), 128, axis=1)
    assert np.array_equal(w, want)


def test_generator_q8_0_encoding_matches_decode():
    rng = np.random.default_rng(6)
    n, k = 3, 128
    codes = rng.integers(-128, 128, (n, k)).astype(np.int8)
    d = rng.uniform(0.0005, 0.0015, (n, k // 32)).astype(np.float16)
    w = oracle.decode(4, synth.encode_q8_0(codes, d), n, k)
    want = codes.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.array_equal(w, want)


def test_generator_q4_k_encoding_matches_decode():
    rng = np.random.default_rng(9)
    n, k = 3, 512
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    sc = rng.integers(0, 64, (n, k // 32)).astype(np.uint8)
    mn = rng.integers(0, 64, (n, k // 32)).astype(np.uint8)
    d = rng.uniform(0.0001, 0.0004, (n, k // 256)).astype(np.float16)
    dmin = rng.uniform(0.0001, 0.0004, (n, k // 256)).astype(np.float16)
    w = oracle.decode(6, synth.encode_q4_k(codes, sc, mn, d, dmin), n, k)
    dd = np.repeat(d.astype(np.float64), 256, axis=1)
    mm = np.repeat(dmin.astype(np.float64), 256, axis=1)
    want = dd * np.repeat(sc, 32, axis=1) * codes - mm * np.repeat(mn, 32, axis=1)
    assert np.array_equal(w, want)


def test_generator_ternary_encoding_matches_decode():
    rng = np.random.default_rng(10)
    n, k = 3, 768
    q = rng.integers(-1, 2, (n, k)).astype(np.int8)
    d = rng.uniform(0.01, 0.03, (n, k // 256)).astype(np.float16)
    w = oracle.decode(7, synth.encode_ternary(q, d), n, k)
    assert np.array_equal(w, q.astype(np.float64) * np.repeat(d.astype(np.float64), 256, axis=1))


def test_generator_ternary_frequencies():
    n, k = 64, 4096
    w = oracle.decode(7, synth.gen_ternary(n, k, 12), n, k)
    q = np.sign(w).astype(np.int64) + 1
    freq = np.bincount(q.reshape(-1), minlength=3) / q.size
    assert np.allclose(freq, synth.TERNARY_PROBS, atol=0.005)


def test_generator_q2_0_code_frequencies():
    canon = synth.gen_q2_0(256, 1024, 11)
    blk = canon.reshape(-1, 34)[:, 2:]
    q = np.stack([(blk >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(-1)
    freq = np.bincount(q, minlength=4) / q.size
    assert np.allclose(freq, synth.Q2_0_PROBS, atol=0.005)


def test_generator_is_deterministic():
    a = synth.gen_q4_0(8, 64, 123)
    b = synth.gen_q4_0(8, 64, 123)
    c = synth.gen_q4_0(8, 64, 124)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(synth.gen_x(4, 64, 1), synth.gen_x(4, 64, 1))


def test_ternary_q2_reads_the_ternary_canonical_format():
    """Codec 8 is a device layout of the ternary codec: the oracle decodes its
    canonical bytes exactly as codec 7's (pinned above by the fixtures)."""
    canon = synth.gen_weight(7, 33, 768, 91)
    assert np.array_equal(oracle.decode(8, canon, 33, 768), oracle.decode(7, canon, 33, 768))
    assert oracle.block_geometry(8) == oracle.block_geometry(7)
