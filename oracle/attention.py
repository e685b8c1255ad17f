"""CPU oracle for attention over a Q8_0 KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the HIP library never calls it and the
two share no code.

What it computes (the plain definition that any FlashAttention reaches up to
rounding; comparison page section 2.3 and the project index, Brick 4: attention
whose K and V come from a Q8_0-compressed cache, dequantized on the fly):

    K, V  = exact fp64 decode of the Q8_0 rows (32-element blocks along the
            head dimension: w = q * d, GGUF block_q8_0 as for the weights)
    S     = scale * Q K^T                    per query head h, with the KV head
            g = h // (H / H_kv)              (grouped-query attention)
    mask  : key s is visible to query m iff s <= (S_len - M) + m when causal
            (the M queries are the last M positions of the S_len tokens)
    P     = softmax over the visible keys of each row, in fp64 (exp of the
            scores minus the row maximum, divided by the row sum)
    O     = P V

Matrix products use numpy's fp64 matmul; there is no tiling, no online
rescaling and no reordering beyond that definition.
"""
from __future__ import annotations

import numpy as np

from . import Q8_0, decode, dequant_f16_bits, f16_to_f64


def q8kv_attention_ref(q16: np.ndarray, k_canon: np.ndarray, v_canon: np.ndarray, kv_heads: int, s_len: int,
                       causal: bool, scale: float, rows=None, kv_f16: bool = False) -> np.ndarray:
    """O [H, len(rows), D] in fp64 for fp16 queries q16 [H, M, D] and canonical
    Q8_0 K, V caches of kv_heads * s_len rows of D elements each.

    kv_f16: use every K and V element rounded once to binary16 (the operand
    precision at which the cache is dequantized for the matrix unit) instead
    of its exact value; everything after that is the same fp64 definition."""
    heads, m, d = q16.shape
    if heads % kv_heads or d % 32 or s_len < m:
        raise ValueError("shape")
    rows = np.arange(m) if rows is None else np.asarray(rows, dtype=np.int64)
    if kv_f16:
        k = f16_to_f64(dequant_f16_bits(Q8_0, k_canon, kv_heads * s_len, d)).reshape(kv_heads, s_len, d)
        v = f16_to_f64(dequant_f16_bits(Q8_0, v_canon, kv_heads * s_len, d)).reshape(kv_heads, s_len, d)
    else:
        k = decode(Q8_0, k_canon, kv_heads * s_len, d).reshape(kv_heads, s_len, d)
        v = decode(Q8_0, v_canon, kv_heads * s_len, d).reshape(kv_heads, s_len, d)
    q = f16_to_f64(np.ascontiguousarray(q16).view(np.uint16))
    group = heads // kv_heads
    offset = s_len - m
    keys = np.arange(s_len)
    out = np.empty((heads, rows.size, d), dtype=np.float64)
    for h in range(heads):
        g = h // group
        scores = (q[h, rows] @ k[g].T) * scale
        if causal:
            visible = keys[None, :] <= (offset + rows)[:, None]
            scores = np.where(visible, scores, -np.inf)
        top = scores.max(axis=1, keepdims=True)
        p = np.exp(scores - top)
        p = p / p.sum(axis=1, keepdims=True)
        out[h] = p @ v[g]
    return out
