"""Byte accounting for KV caches and for one decode step.

The KV footprint per token is two tensors (K and V) times layers times KV
heads times head dimension times bytes per element ("vLLM &
High-Throughput Serving", section 1, memory-per-token equation; "How LLM
Inference Engines Work", KV cache per layer formula).  "AI Inference
Serving at Scale", section 2, writes a formula with one more factor of 2,
but its own 2.6 MB-per-token figure omits that factor; the figures, not
the garbled formula, are what the tests pin.

``decode_bytes`` / ``write_bytes`` give the algorithmic HBM traffic of one
launch: every byte the operation must read or write at least once.
"""

from __future__ import annotations

import numpy as np

ELEMENT_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1, "fp8_e5m2": 1}


def row_bytes(cache_dtype: str, head_dim: int) -> int:
    """Bytes of one token's K (or V) row of one KV head in the cache.  An
    INT4 row is head_dim 4-bit codes plus its own float32 scale."""
    if cache_dtype == "int4":
        return head_dim // 2 + 4
    return head_dim * ELEMENT_BYTES[cache_dtype]


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int,
                       bytes_per_element: int) -> int:
    """K and V bytes one token occupies across all layers."""
    return 2 * layers * kv_heads * head_dim * bytes_per_element


def kv_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int,
             bytes_per_element: int) -> int:
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim,
                                       bytes_per_element)


def decode_bytes(context_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, cache_dtype: str,
                 q_dtype: str) -> dict:
    """Algorithmic bytes of one decode over a batch (one layer).

    K and V of every valid token, each read once; q read and out written
    once; the used block-table entries and the lengths read once; one
    float32 scale per KV head for K and for V when the cache is FP8 (an
    INT4 cache's per-token scales are part of its rows).
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    qb = ELEMENT_BYTES[q_dtype]
    tokens = int(lens.sum())
    kv = tokens * 2 * num_kv_heads * row_bytes(cache_dtype, head_dim)
    s = len(lens)
    q_out = 2 * s * num_q_heads * head_dim * qb
    tables = int((-(-lens // block_size)).sum()) * 4 + s * 4
    scales = 2 * num_kv_heads * 4 if cache_dtype.startswith("fp8") else 0
    return {"kv": kv, "q_out": q_out, "tables": tables, "scales": scales,
            "total": kv + q_out + tables + scales, "tokens": tokens}


def write_bytes(num_tokens: int, num_kv_heads: int, head_dim: int,
                src_dtype: str, cache_dtype: str) -> int:
    """Algorithmic bytes of one cache append: read new rows, write slots."""
    rows = num_tokens * 2 * num_kv_heads
    return (rows * head_dim * ELEMENT_BYTES[src_dtype] + rows * row_bytes(cache_dtype, head_dim)
            + num_tokens * 8)


def copy_bytes(num_pairs: int, num_kv_heads: int, head_dim: int, block_size: int,
               cache_dtype: str) -> int:
    """Algorithmic bytes of a block copy: each pair reads and writes one
    block of the K pool and one of the V pool (every KV head)."""
    block = num_kv_heads * block_size * row_bytes(cache_dtype, head_dim)
    return num_pairs * 2 * 2 * block + num_pairs * 16


def prefill_bytes(context_lens, query_lens, num_q_heads: int, num_kv_heads: int,
                  head_dim: int, block_size: int, cache_dtype: str, q_dtype: str) -> dict:
    """Algorithmic bytes and flops of attention for several query tokens per
    sequence: every sequence's cached K and V read once, q read and out
    written once, the used table entries; flops 4 * head_dim per (query
    row, query head, visible token) -- q.k and the weighted V sum, 2 flops
    per multiply-add -- with row i of a Q-token chunk seeing L - Q + i + 1
    tokens."""
    lens = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    qb = ELEMENT_BYTES[q_dtype]
    tokens = int(lens.sum())
    kv = tokens * 2 * num_kv_heads * row_bytes(cache_dtype, head_dim)
    rows = int(ql.sum())
    q_out = 2 * rows * num_q_heads * head_dim * qb
    tables = int((-(-lens // block_size)).sum()) * 4 + len(lens) * 8
    visible = int((ql * (lens - ql) + ql * (ql + 1) // 2).sum())  # sum over rows of (p + 1)
    flops = 4 * head_dim * num_q_heads * visible
    return {"kv": kv, "q_out": q_out, "tables": tables, "total": kv + q_out + tables,
            "flops": flops, "query_rows": rows, "tokens": tokens}
