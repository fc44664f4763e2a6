"""Full and sparse decode attention, float64 (oracle; test infrastructure only).

Full attention is what layers 0-1 and every delta-layer compute ("Methodology in
Plain English": the early layers and the delta-layers attend to the whole
context).  Sparse attention is the same softmax attention restricted to the
tokens of the chosen pages (same section); the softmax renormalises over those
tokens.

Readings where the pages are silent:
* grouped-query attention: query head h reads KV head g(h) = floor(h / G),
  G = Hq / Hkv (consecutive query heads share a KV head);
* the softmax scale ``sm_scale`` is an argument (logit = sm_scale * <q, k>);
* the token appended this step is part of the context (length T includes it);
* LSE is the natural-log log-sum-exp of the scaled logits.
"""
from __future__ import annotations

import numpy as np


def attention_over_tokens(q_h: np.ndarray, K_g: np.ndarray, V_g: np.ndarray, sm_scale: float):
    """Softmax attention of one query head over a set of tokens.

    q_h [D], K_g/V_g [N, D] (float64).  Returns (out [D], lse, p [N], logits [N]).
    Computed with the usual max shift: p = exp(s - max s) / sum exp(s - max s).
    """
    s = sm_scale * (K_g @ q_h)
    if s.size == 0:
        return np.zeros(V_g.shape[1]), -np.inf, s, s
    m = np.max(s)
    e = np.exp(s - m)
    denom = np.sum(e)
    p = e / denom
    out = p @ V_g
    return out, m + np.log(denom), p, s


def full_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Full decode attention for one sequence.

    q [Hq, D]; K, V [Hkv, T, D].  Returns (out [Hq, D], lse [Hq], p [Hq, T]).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, d = q.shape
    hkv, T, _ = K.shape
    G = hq // hkv
    out = np.zeros((hq, d))
    lse = np.zeros(hq)
    p = np.zeros((hq, T))
    for h in range(hq):
        g = h // G
        out[h], lse[h], p[h], _ = attention_over_tokens(q[h], K[g], V[g], sm_scale)
    return out, lse, p


def selected_tokens(sel_pages, T: int, page: int) -> np.ndarray:
    """Token positions t < T whose page floor(t / page) is in ``sel_pages`` (ascending)."""
    pages = np.asarray(sorted(set(int(j) for j in sel_pages)), dtype=np.int64)
    if pages.size == 0:
        return np.zeros(0, dtype=np.int64)
    toks = (pages[:, None] * page + np.arange(page)[None, :]).reshape(-1)
    return toks[toks < T]


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sel, page: int, sm_scale: float):
    """Sparse decode attention for one sequence.

    ``sel`` is a list of Hkv page lists (one per KV head, logical page ids), or a
    single list shared by every KV head.  Returns (out [Hq, D], lse [Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, d = q.shape
    hkv, T, _ = K.shape
    G = hq // hkv
    if len(sel) > 0 and np.isscalar(sel[0]):
        sel = [sel] * hkv
    out = np.zeros((hq, d))
    lse = np.zeros(hq)
    for h in range(hq):
        g = h // G
        toks = selected_tokens(sel[g], T, page)
        out[h], lse[h], _, _ = attention_over_tokens(q[h], K[g][toks], V[g][toks], sm_scale)
    return out, lse
