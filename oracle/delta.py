"""Delta-layer page scoring and page selection, float64 (oracle; test infrastructure only).

Steps, in the order of "Methodology in Plain English" on the DELTA AI summary page:
1. full attention of the delta-layer gives each head's softmax weights p[h, t];
2. per-token score: the token's largest softmax weight over the heads;
3. tokens are grouped into fixed-size pages (page size P);
4. page score: sum of the per-token scores of the page;
5. the most recent pages are kept as a recency window (L pages, "Main Findings");
6. the remaining budget (K pages) goes to the older pages of largest score.

Readings where the pages are silent, ambiguous or at odds:
* heads aggregated (scope "group"): the query heads of one KV group, giving one
  selection per KV head; scope "all": every query head, one selection per
  sequence shared by all KV heads.  The pages say "across heads" without an index;
* aggregation operator: "max" (the pages' rule); "sum" is offered because one
  workload description speaks of a group-summed score;
* recency window: the last L pages, page-granular, the partial last page
  included; the K top pages are taken among the older pages only, so the result
  has min(NP, K + L) pages;
* a partial last page scores only its valid tokens;
* ties at the K-th score: the lower page index wins (key (-score, index));
* the selection is returned as ascending logical page indices.
"""
from __future__ import annotations

import numpy as np

from .attention import full_attention


def token_scores(p: np.ndarray, hkv: int, agg: str = "max", scope: str = "group") -> np.ndarray:
    """Per-token scores from softmax weights p [Hq, T].

    scope "group": returns [Hkv, T], row g aggregates heads g*G .. g*G+G-1.
    scope "all":   returns [1, T], aggregating every head.
    """
    p = np.asarray(p, dtype=np.float64)
    hq, T = p.shape
    G = hq // hkv
    groups = [list(range(g * G, (g + 1) * G)) for g in range(hkv)] if scope == "group" else [list(range(hq))]
    out = np.zeros((len(groups), T))
    for r, heads in enumerate(groups):
        out[r] = np.max(p[heads], axis=0) if agg == "max" else np.sum(p[heads], axis=0)
    return out


def page_scores(a: np.ndarray, page: int) -> np.ndarray:
    """Page scores from per-token scores a [R, T]: S[r, j] = sum of a[r, t] over the
    valid tokens t of page j (t in [j*P, min((j+1)*P, T)))."""
    a = np.asarray(a, dtype=np.float64)
    R, T = a.shape
    NP = -(-T // page)
    S = np.zeros((R, NP))
    for r in range(R):
        for j in range(NP):
            S[r, j] = np.sum(a[r, j * page: min((j + 1) * page, T)])
    return S


def select_pages(S_row, k_top: int, recency: int) -> list:
    """Selection for one score row S_row [NP].

    Recency window R = the last ``recency`` pages; candidates C = the older pages;
    Top = the ``k_top`` candidates of largest score, ties to the lower index.
    Returns sorted(R u Top).
    """
    S_row = [float(x) for x in S_row]
    NP = len(S_row)
    first_recent = max(0, NP - recency)
    recent = list(range(first_recent, NP))
    candidates = list(range(0, first_recent))
    ranked = sorted(candidates, key=lambda j: (-S_row[j], j))
    top = ranked[: min(k_top, len(candidates))]
    return sorted(recent + top)


def delta_layer(q, K, V, sm_scale: float, page: int, k_top: int, recency: int,
                agg: str = "max", scope: str = "group"):
    """One delta-layer: full attention output plus the page selection it installs.

    Returns dict(out [Hq, D], lse [Hq], p [Hq, T], token_scores, page_scores, sel)
    where ``sel`` is a list with one ascending page list per score row
    (Hkv rows for scope "group", one row for scope "all").
    """
    out, lse, p = full_attention(q, K, V, sm_scale)
    hkv = np.asarray(K).shape[0]
    a = token_scores(p, hkv, agg, scope)
    S = page_scores(a, page)
    sel = [select_pages(S[r], k_top, recency) for r in range(S.shape[0])]
    return dict(out=out, lse=lse, p=p, token_scores=a, page_scores=S, sel=sel)
