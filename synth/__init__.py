"""Seeded synthetic inputs for the quantized prefill GEMM path.

This module only draws random numbers and lays them out in the canonical
byte formats of the weight codecs.  It performs no dequantization and
no products: decoding and contraction belong to the oracle (``oracle/``) and
to the HIP library, which share nothing but these inputs.

Canonical byte formats (the input contract both sides read):

* Q4_0 (GGUF block_q4_0, named on the project index page, Table B): blocks of
  32 weights along K, 18 bytes each: little-endian fp16 scale ``d`` in bytes
  0-1, then 16 bytes where byte ``j`` carries weight ``j`` in its low nibble
  and weight ``j + 16`` in its high nibble.  Weight value ``(q - 8) * d``.
* MLX4-G64 (MLX-style 4-bit affine, group 64 along K): three consecutive
  arrays: codes as little-endian uint32 words ``[N, K/8]`` holding 8 codes,
  element 0 in the low 4 bits; then fp16 scales ``[N, K/64]``; then fp16
  biases ``[N, K/64]``.  Weight value ``q * s + b``.
* Q2_0 (PrismML block_prism_q2_0, releases page, v0.3.0 "PrismML Q2_0
  Ternary Codec"): blocks of 128 weights, 34 bytes: fp16 ``d`` in bytes 0-1,
  then 32 bytes of 2-bit codes, weight ``i`` in byte ``2 + i // 4`` at bit
  ``2 * (i % 4)``.  Weight value ``(q - 1) * d``.
* MLX4-G32: as MLX4-G64 with one scale and bias per 32 weights (the group of
  the pages' 20-byte block_mlx_4bit, comparison page section 4).
* Q8_0 (GGUF block_q8_0; the registry of the releases page, v0.3.0, lists Q8_0
  without a layout): blocks of 32 weights, 34 bytes: fp16 ``d`` in bytes 0-1,
  then weight ``j`` as the two's-complement byte ``2 + j``.  Weight value
  ``q * d``.
* Q4_K (GGUF super-block; the pages list "Q4_K (GGUF Super-Blocks)" among the
  router's formats without a layout, so this is the public GGUF layout):
  256 weights in 144 bytes: fp16 ``d`` (bytes 0-1), fp16 ``dmin`` (2-3), 12
  bytes of 6-bit sub-block scales ``sc[j]`` and mins ``m[j]`` (4-15), then 128
  code bytes in four 32-byte runs, byte ``l`` of run ``c`` holding weight
  ``64 c + l`` (low nibble) and ``64 c + 32 + l`` (high nibble).  For
  ``j < 4``: byte ``4 + j`` = ``sc[j]`` plus the top two bits of ``sc[j + 4]``
  at bits 6-7, byte ``8 + j`` = ``m[j]`` plus the top two bits of ``m[j + 4]``;
  byte ``12 + j`` = low nibbles of ``sc[j + 4]`` and ``m[j + 4]``.  Weight
  value ``d * sc[j] * q - dmin * m[j]`` in sub-block ``j`` (32 weights).
* Ternary 1.58-bit (the pages name the BitNet ternary format without a
  packing; reading): 256 weights in 54 bytes: fp16 ``d`` (bytes 0-1), then
  byte ``2 + j`` holding weights ``5 j .. 5 j + 4`` as base-3 digits
  ``t = q + 1`` (weight ``5 j + i`` contributes ``t * 3**i``); weight 255 is
  digit 0 of byte 53.  Weight value ``q * d`` with ``q`` in {-1, 0, +1}.

Distributions and shapes follow the five workloads of the method: fp16
activations ~N(0,1); Q4_0 scales ~U(0.005, 0.02) with codes ~U{0..15}; MLX
scales ~U(0.002, 0.01), biases ~N(0, 0.02), codes ~U{0..15}; Q2_0 scales
~U(0.01, 0.05) with P(q=0,1,2,3) = 0.30, 0.35, 0.30, 0.05.  The Q8_0 workload
(a next-step codec, not one of the five) uses codes ~U{-127..127} and scales
~U(0.0005, 0.0015), which keeps its weights in the Q4_0 workload's range.
The Q4_K workloads (next-step codec) draw codes ~U{0..15}, sub-block scales
and mins ~U{0..63} and super-block d, dmin ~U(0.0001, 0.0004).  The ternary
workloads draw q = -1, 0, +1 with probabilities 0.345, 0.31, 0.345 (absmean
rounding of Gaussian weights gives about 0.31 zeros) and d ~U(0.01, 0.03).

Random streams: numpy PCG64 seeded from ``SeedSequence([seed, tensor_id])``
so every tensor of every workload has its own reproducible stream.
"""
from __future__ import annotations

import dataclasses

import numpy as np

CODEC_Q4_0 = 1
CODEC_MLX4_G64 = 2
CODEC_Q2_0 = 3
CODEC_Q8_0 = 4
CODEC_MLX4_G32 = 5
CODEC_Q4_K = 6
CODEC_TERNARY = 7
CODEC_TERNARY_Q2 = 8     # the ternary canonical format, held on the device as 2-bit codes

CODEC_NAMES = {CODEC_Q4_0: "q4_0", CODEC_MLX4_G64: "mlx4_g64", CODEC_Q2_0: "q2_0", CODEC_Q8_0: "q8_0",
               CODEC_MLX4_G32: "mlx4_g32", CODEC_Q4_K: "q4_k",
               CODEC_TERNARY: "ternary", CODEC_TERNARY_Q2: "ternary_q2"}
# weights per block (scale group) along K
BLOCK = {CODEC_Q4_0: 32, CODEC_MLX4_G64: 64, CODEC_Q2_0: 128, CODEC_Q8_0: 32, CODEC_MLX4_G32: 32, CODEC_Q4_K: 256,
         CODEC_TERNARY: 256, CODEC_TERNARY_Q2: 256}

BASE_SEED = 0x51C0DEC0

# tensor ids inside one workload seed
T_X, T_W, T_WG, T_WU = 1, 2, 3, 4


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed & 0xFFFFFFFF, tensor_id])))


def canonical_bytes(codec: int, n: int, k: int) -> int:
    """Size in bytes of the canonical encoding of an [n, k] weight matrix."""
    b = BLOCK[codec]
    if k % b:
        raise ValueError(f"K={k} is not a multiple of the {CODEC_NAMES[codec]} block {b}")
    if codec == CODEC_Q4_0:
        return n * (k // 32) * 18
    if codec == CODEC_MLX4_G64:
        return n * (k // 2) + 2 * (n * (k // 64) * 2)
    if codec == CODEC_MLX4_G32:
        return n * (k // 2) + 2 * (n * (k // 32) * 2)
    if codec == CODEC_Q2_0:
        return n * (k // 128) * 34
    if codec == CODEC_Q8_0:
        return n * (k // 32) * 34
    if codec == CODEC_Q4_K:
        return n * (k // 256) * 144
    if codec in (CODEC_TERNARY, CODEC_TERNARY_Q2):
        return n * (k // 256) * 54
    raise ValueError(codec)


def fp16_uniform(rng: np.random.Generator, lo: float, hi: float, size) -> np.ndarray:
    return (lo + (hi - lo) * rng.random(size)).astype(np.float16)


def gen_x(m: int, k: int, seed: int, tensor_id: int = T_X) -> np.ndarray:
    """fp16 activations [m, k] drawn from N(0, 1) and rounded to fp16."""
    return _rng(seed, tensor_id).standard_normal((m, k)).astype(np.float16)


def encode_q4_0(codes: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Lay out codes [n, k] (uint8 0..15) and fp16 scales [n, k/32] as Q4_0 blocks."""
    n, k = codes.shape
    nb = k // 32
    q = codes.reshape(n, nb, 32).astype(np.uint8)
    out = np.empty((n, nb, 18), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:18] = q[:, :, 0:16] | (q[:, :, 16:32] << 4)
    return out.reshape(-1)


def encode_mlx4(codes: np.ndarray, s: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Lay out codes [n, k] (0..15), fp16 scales and biases [n, k/group] in MLX order."""
    n, k = codes.shape
    q = codes.reshape(n, k // 8, 8).astype(np.uint32)
    words = np.zeros((n, k // 8), dtype=np.uint32)
    for e in range(8):
        words |= q[:, :, e] << np.uint32(4 * e)
    parts = [words.astype("<u4").view(np.uint8).reshape(-1),
             s.astype("<f2").view(np.uint8).reshape(-1),
             b.astype("<f2").view(np.uint8).reshape(-1)]
    return np.concatenate(parts)


def encode_q2_0(codes: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Lay out codes [n, k] (0..3) and fp16 scales [n, k/128] as Q2_0 blocks."""
    n, k = codes.shape
    nb = k // 128
    q = codes.reshape(n, nb, 32, 4).astype(np.uint8)
    out = np.empty((n, nb, 34), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:34] = q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)
    return out.reshape(-1)


def encode_q8_0(codes: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Lay out codes [n, k] (int8) and fp16 scales [n, k/32] as Q8_0 blocks."""
    n, k = codes.shape
    nb = k // 32
    out = np.empty((n, nb, 34), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:34] = codes.astype(np.int8).reshape(n, nb, 32).view(np.uint8)
    return out.reshape(-1)


def encode_q4_k(codes: np.ndarray, sc: np.ndarray, mn: np.ndarray, d: np.ndarray,
                dmin: np.ndarray) -> np.ndarray:
    """Lay out codes [n, k] (0..15), 6-bit sub-block scales and mins [n, k/32]
    (0..63) and fp16 super-block d, dmin [n, k/256] as Q4_K super-blocks."""
    n, k = codes.shape
    nb = k // 256
    s = sc.reshape(n, nb, 8).astype(np.uint8)
    m = mn.reshape(n, nb, 8).astype(np.uint8)
    q = codes.reshape(n, nb, 4, 2, 32).astype(np.uint8)      # run, nibble half, byte
    out = np.empty((n, nb, 144), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:4] = dmin.astype("<f2").reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 4:8] = (s[:, :, 0:4] & 63) | ((s[:, :, 4:8] >> 4) << 6)
    out[:, :, 8:12] = (m[:, :, 0:4] & 63) | ((m[:, :, 4:8] >> 4) << 6)
    out[:, :, 12:16] = (s[:, :, 4:8] & 15) | ((m[:, :, 4:8] & 15) << 4)
    out[:, :, 16:144] = (q[:, :, :, 0, :] | (q[:, :, :, 1, :] << 4)).reshape(n, nb, 128)
    return out.reshape(-1)


def encode_ternary(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Lay out ternary values q [n, k] (-1, 0, +1) and fp16 scales [n, k/256] as
    54-byte blocks of base-3 digits."""
    n, k = q.shape
    nb = k // 256
    t = (q.astype(np.int64) + 1).reshape(n, nb, 256)
    padded = np.zeros((n, nb, 260), dtype=np.int64)
    padded[:, :, :256] = t
    digits = padded.reshape(n, nb, 52, 5)
    packed = np.zeros((n, nb, 52), dtype=np.int64)
    for i in range(5):
        packed += digits[:, :, :, i] * 3 ** i
    out = np.empty((n, nb, 54), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:54] = packed.astype(np.uint8)
    return out.reshape(-1)


TERNARY_PROBS = (0.345, 0.31, 0.345)


def gen_ternary(n: int, k: int, seed: int, tensor_id: int = T_W,
                d_range=(0.01, 0.03), probs=TERNARY_PROBS) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    u = rng.random((n, k))
    edges = np.cumsum(np.asarray(probs, dtype=np.float64))[:-1]
    q = np.searchsorted(edges, u, side="right").astype(np.int8) - 1
    d = fp16_uniform(rng, d_range[0], d_range[1], (n, k // 256))
    return encode_ternary(q, d)


def gen_q4_0(n: int, k: int, seed: int, tensor_id: int = T_W,
             d_range=(0.005, 0.02)) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    d = fp16_uniform(rng, d_range[0], d_range[1], (n, k // 32))
    return encode_q4_0(codes, d)


def gen_mlx4(n: int, k: int, seed: int, tensor_id: int = T_W,
             s_range=(0.002, 0.01), b_sigma=0.02) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    s = fp16_uniform(rng, s_range[0], s_range[1], (n, k // 64))
    b = (b_sigma * rng.standard_normal((n, k // 64))).astype(np.float16)
    return encode_mlx4(codes, s, b)


def gen_mlx4_g32(n: int, k: int, seed: int, tensor_id: int = T_W,
                 s_range=(0.002, 0.01), b_sigma=0.02) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    s = fp16_uniform(rng, s_range[0], s_range[1], (n, k // 32))
    b = (b_sigma * rng.standard_normal((n, k // 32))).astype(np.float16)
    return encode_mlx4(codes, s, b)


Q2_0_PROBS = (0.30, 0.35, 0.30, 0.05)


def gen_q2_0(n: int, k: int, seed: int, tensor_id: int = T_W,
             d_range=(0.01, 0.05), probs=Q2_0_PROBS) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    u = rng.random((n, k))
    edges = np.cumsum(np.asarray(probs, dtype=np.float64))[:-1]
    codes = np.searchsorted(edges, u, side="right").astype(np.uint8)
    d = fp16_uniform(rng, d_range[0], d_range[1], (n, k // 128))
    return encode_q2_0(codes, d)


def gen_q8_0(n: int, k: int, seed: int, tensor_id: int = T_W,
             d_range=(0.0005, 0.0015)) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    codes = rng.integers(-127, 128, size=(n, k), dtype=np.int16).astype(np.int8)
    d = fp16_uniform(rng, d_range[0], d_range[1], (n, k // 32))
    return encode_q8_0(codes, d)


def gen_q4_k(n: int, k: int, seed: int, tensor_id: int = T_W,
             d_range=(0.0001, 0.0004)) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(n, k // 32), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(n, k // 32), dtype=np.uint8)
    d = fp16_uniform(rng, d_range[0], d_range[1], (n, k // 256))
    dmin = fp16_uniform(rng, d_range[0], d_range[1], (n, k // 256))
    return encode_q4_k(codes, sc, mn, d, dmin)


GEN = {CODEC_Q4_0: gen_q4_0, CODEC_MLX4_G64: gen_mlx4, CODEC_Q2_0: gen_q2_0, CODEC_Q8_0: gen_q8_0,
       CODEC_MLX4_G32: gen_mlx4_g32, CODEC_Q4_K: gen_q4_k, CODEC_TERNARY: gen_ternary,
       CODEC_TERNARY_Q2: gen_ternary}


def gen_weight(codec: int, n: int, k: int, seed: int, tensor_id: int = T_W) -> np.ndarray:
    return GEN[codec](n, k, seed, tensor_id)


GATED = ("swiglu", "geglu")     # gate/up pairs with a gated epilogue


@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the five workloads: shapes, codec and which entry point runs it."""
    name: str
    op: str          # "prefill" | "heads" | "swiglu" | "geglu" | "gemv"
    codec: int
    m: int
    k: int
    n: int
    seed: int
    head_dim: int = 0   # "heads": Y written as [N / head_dim, M, head_dim]

    def x(self) -> np.ndarray:
        return gen_x(self.m, self.k, self.seed)

    def weights(self):
        if self.op in GATED:
            return (gen_weight(self.codec, self.n, self.k, self.seed, T_WG),
                    gen_weight(self.codec, self.n, self.k, self.seed, T_WU))
        return (gen_weight(self.codec, self.n, self.k, self.seed, T_W),)

    def flops(self) -> int:
        mats = 2 if self.op in GATED else 1
        return 2 * self.m * self.n * self.k * mats

    def algorithmic_bytes(self) -> int:
        mats = 2 if self.op in GATED else 1
        return mats * canonical_bytes(self.codec, self.n, self.k) + 2 * self.m * self.k + 2 * self.m * self.n


WORKLOADS = {
    "q4_0_tiny_16x256x256": Workload("q4_0_tiny_16x256x256", "prefill", CODEC_Q4_0, 16, 256, 256, BASE_SEED + 1),
    "q4_0_prefill_2048x2048x8192": Workload("q4_0_prefill_2048x2048x8192", "prefill", CODEC_Q4_0, 2048, 2048, 8192, BASE_SEED + 2),
    "mlx4_swiglu_2048x4096x14336": Workload("mlx4_swiglu_2048x4096x14336", "swiglu", CODEC_MLX4_G64, 2048, 4096, 14336, BASE_SEED + 3),
    "q2_0_prefill_2048x4096x4096": Workload("q2_0_prefill_2048x4096x4096", "prefill", CODEC_Q2_0, 2048, 4096, 4096, BASE_SEED + 4),
    "q4_0_gemv_1x4096x14336": Workload("q4_0_gemv_1x4096x14336", "gemv", CODEC_Q4_0, 1, 4096, 14336, BASE_SEED + 5),
    "q4_0_gemv_64x4096x14336": Workload("q4_0_gemv_64x4096x14336", "gemv", CODEC_Q4_0, 64, 4096, 14336, BASE_SEED + 5),
    # next-step codec on the 1B-shape up-projection
    "q8_0_prefill_2048x2048x8192": Workload("q8_0_prefill_2048x2048x8192", "prefill", CODEC_Q8_0, 2048, 2048, 8192, BASE_SEED + 6),
    # next-step codec variant: MLX 4-bit with group 32 on the 1B-shape up-projection
    "mlx4_g32_prefill_2048x2048x8192": Workload("mlx4_g32_prefill_2048x2048x8192", "prefill", CODEC_MLX4_G32, 2048, 2048,
                                                8192, BASE_SEED + 9),
    # next-step layout: 8B-shape Q projection written per head ([32, 2048, 128])
    "q4_0_qproj_heads_2048x4096x4096": Workload("q4_0_qproj_heads_2048x4096x4096", "heads", CODEC_Q4_0, 2048, 4096, 4096,
                                                BASE_SEED + 8, head_dim=128),
    # next-step epilogue: the 8B-shape gate/up pair with GeGLU instead of SwiGLU
    "mlx4_geglu_2048x4096x14336": Workload("mlx4_geglu_2048x4096x14336", "geglu", CODEC_MLX4_G64, 2048, 4096, 14336, BASE_SEED + 7),
    # next-step codec: GGUF Q4_K super-blocks on the 1B-shape up-projection and the 8B decode shape
    "q4_k_prefill_2048x2048x8192": Workload("q4_k_prefill_2048x2048x8192", "prefill", CODEC_Q4_K, 2048, 2048, 8192,
                                            BASE_SEED + 10),
    "q4_k_gemv_1x4096x14336": Workload("q4_k_gemv_1x4096x14336", "gemv", CODEC_Q4_K, 1, 4096, 14336, BASE_SEED + 11),
    # next-step codec: BitNet ternary (base-3, 1.6875 bits per weight) on the same two shapes
    "ternary_prefill_2048x2048x8192": Workload("ternary_prefill_2048x2048x8192", "prefill", CODEC_TERNARY, 2048, 2048,
                                               8192, BASE_SEED + 12),
    "ternary_gemv_1x4096x14336": Workload("ternary_gemv_1x4096x14336", "gemv", CODEC_TERNARY, 1, 4096, 14336,
                                          BASE_SEED + 13),
    # the same ternary inputs held on the device as 2-bit codes (the Q2_0 planar format)
    "ternary_q2_prefill_2048x2048x8192": Workload("ternary_q2_prefill_2048x2048x8192", "prefill", CODEC_TERNARY_Q2, 2048,
                                                  2048, 8192, BASE_SEED + 12),
    "ternary_q2_gemv_1x4096x14336": Workload("ternary_q2_gemv_1x4096x14336", "gemv", CODEC_TERNARY_Q2, 1, 4096, 14336,
                                             BASE_SEED + 13),
}


T_Q, T_K, T_V = 5, 6, 7


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """Attention over a Q8_0 KV cache: H query heads of M queries attend to
    the S positions of KV heads shared by H / H_kv query heads each."""
    name: str
    heads: int
    kv_heads: int
    m: int
    s: int
    head_dim: int
    causal: bool
    seed: int

    def q(self) -> np.ndarray:
        """fp16 queries [H, M, D] ~N(0, 1)."""
        return gen_x(self.heads * self.m, self.head_dim, self.seed, T_Q).reshape(self.heads, self.m, self.head_dim)

    def kv(self):
        """Canonical Q8_0 rows [H_kv * S, D] of K and of V: codes ~U{-127..127},
        block scales ~U(0.01, 0.03), so elements spread over about +-3.8."""
        rows = self.kv_heads * self.s
        return (gen_q8_0(rows, self.head_dim, self.seed, T_K, d_range=(0.01, 0.03)),
                gen_q8_0(rows, self.head_dim, self.seed, T_V, d_range=(0.01, 0.03)))

    def visible_pairs(self) -> int:
        if not self.causal:
            return self.m * self.s
        off = self.s - self.m
        return sum(off + i + 1 for i in range(self.m))

    def flops(self) -> int:
        """2 D for the score and 2 D for the weighted sum of every visible (query, key) pair."""
        return 4 * self.head_dim * self.heads * self.visible_pairs()

    def algorithmic_bytes(self) -> int:
        """Q and O in fp16 once, K and V as canonical Q8_0 once."""
        cache = 2 * self.kv_heads * self.s * (self.head_dim // 32) * 34
        return 2 * 2 * self.heads * self.m * self.head_dim + cache


ATTN_WORKLOADS = {
    # 8B-shape prefill attention: 32 query heads over 8 KV heads (grouped 4:1), D = 128, 2048 tokens, causal
    "q8kv_attention_2048x2048_h32kv8_d128": AttnWorkload("q8kv_attention_2048x2048_h32kv8_d128", 32, 8, 2048, 2048, 128,
                                                         True, BASE_SEED + 20),
    # 1B-shape prefill attention: 32 heads, D = 64
    "q8kv_attention_2048x2048_h32kv8_d64": AttnWorkload("q8kv_attention_2048x2048_h32kv8_d64", 32, 8, 2048, 2048, 64,
                                                        True, BASE_SEED + 21),
}
