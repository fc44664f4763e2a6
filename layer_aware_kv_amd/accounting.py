"""Algorithmic byte and token counts of the decode-attention tiers.

These are the bytes each tier must move, not what the hardware moved:
  full layer   : sum_b T_b * Hkv * D * 2 * e      (K and V of every token, read once per KV head)
                 + 2 * B * Hq * D * e             (q read, out written)
  delta layer  : full + B * R * (k + L) * 4       (the selection written)
  sparse layer : sum_{b,g} U_{b,g} * D * 2 * e    (U = valid tokens of the selected pages)
                 + 2 * B * Hq * D * e + B * R * (k + L) * 4   (q, out, selection read)
  append       : 2 * B * Hkv * D * e
The delta-layer's logits / page-score scratch is reported separately as overhead.
``kv_row`` (optional everywhere) is the bytes of one token's K (or V) row of one KV
head when the pool's element differs from the activations' (fp8 pools: D one-byte
codes plus a 4-byte scale); it defaults to D * e.
"""
from __future__ import annotations

import math


def kv_cache_bytes(layers, kv_heads, head_dim, tokens, batch, elem_bytes):
    """Bytes of a whole KV cache (K and V of every layer, head and token)."""
    return 2 * layers * kv_heads * head_dim * tokens * batch * elem_bytes


def kv_row_bytes(d, kv_dtype):
    """Bytes of one token's K (or V) row of one KV head in a pool of ``kv_dtype``."""
    return {"bf16": 2 * d, "f32": 4 * d, "fp8": d + 4}[kv_dtype]


def full_layer_bytes(lengths, hq, hkv, d, e, kv_row=None):
    row = d * e if kv_row is None else kv_row
    return sum(int(t) for t in lengths) * hkv * row * 2 + 2 * len(lengths) * hq * d * e


def delta_layer_bytes(lengths, hq, hkv, d, e, k_top, recency, rows_per_seq=None, kv_row=None):
    R = hkv if rows_per_seq is None else rows_per_seq
    return full_layer_bytes(lengths, hq, hkv, d, e, kv_row) + len(lengths) * R * (k_top + recency) * 4


def delta_scratch_bytes(lengths, hq, hkv, page):
    """Logits written + read, page scores written + read (float32)."""
    toks = sum(int(t) for t in lengths)
    pages = sum(math.ceil(int(t) / page) for t in lengths)
    return 2 * 4 * hq * toks + 2 * 4 * hkv * pages


def selected_tokens(T, page, k_top, recency):
    """Valid tokens a full selection covers: min(NP, k + L) pages, the partial last page
    (always in the recency window when recency >= 1) counted by its valid tokens."""
    NP = math.ceil(T / page)
    n = min(NP, k_top + recency)
    if n == 0:
        return 0
    last = T - (NP - 1) * page
    if recency >= 1:
        return (n - 1) * page + last
    return n * page if n < NP else (n - 1) * page + last


def sparse_layer_bytes(lengths, hq, hkv, d, e, page, k_top, recency, rows_per_seq=None, kv_row=None):
    R = hkv if rows_per_seq is None else rows_per_seq
    row = d * e if kv_row is None else kv_row
    toks = sum(selected_tokens(int(t), page, k_top, recency) for t in lengths)
    return toks * hkv * row * 2 + 2 * len(lengths) * hq * d * e + len(lengths) * R * (k_top + recency) * 4


def append_bytes(batch, hkv, d, e, kv_row=None):
    """Rows read (activations) plus rows written (pool)."""
    row = d * e if kv_row is None else kv_row
    return 2 * batch * hkv * d * e if kv_row is None else batch * hkv * 2 * (d * e + row)


def attended_tokens(lengths, tiers, page, k_top, recency):
    """Tokens attended per step summed over layers (per KV head)."""
    tot = 0
    for tier in tiers:
        for t in lengths:
            tot += int(t) if tier != "sparse" else selected_tokens(int(t), page, k_top, recency)
    return tot


def stack_bytes(lengths, tiers, hq, hkv, d, e, page, k_top, recency, kv_row=None):
    """Algorithmic bytes of one decode step of the stack, split by tier."""
    out = {"full": 0, "delta": 0, "sparse": 0, "append": 0}
    for tier in tiers:
        out["append"] += append_bytes(len(lengths), hkv, d, e, kv_row)
        if tier == "full":
            out["full"] += full_layer_bytes(lengths, hq, hkv, d, e, kv_row)
        elif tier == "delta":
            out["delta"] += delta_layer_bytes(lengths, hq, hkv, d, e, k_top, recency, kv_row=kv_row)
        else:
            out["sparse"] += sparse_layer_bytes(lengths, hq, hkv, d, e, page, k_top, recency, kv_row=kv_row)
    return out
