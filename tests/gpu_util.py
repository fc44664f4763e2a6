"""Shared helpers of the GPU parity tests (device set-up, comparisons with the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workload import philox as px

TOL = {"bf16": 2e-2, "f32": 1e-4}       # max-abs output error
LSE_TOL = {"bf16": 1e-3, "f32": 1e-4}
BAND = 1e-3                              # relative selection boundary band
F32_MIN_NORMAL = 2.0 ** -126


def tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdtype(dtype)).cuda().contiguous()


def make_cache(case, page, num_layers=1, extra_tokens=1, spare_pages=4):
    """Cache holding ``case`` (prefilled to lengths - 1, then one decode step appends the last
    token), so that attention runs right after an append, as in decode."""
    from layer_aware_kv_amd import PagedKVCache
    B, HQ, D = case.q.shape
    HKV = case.K.shape[1]
    lens = case.lengths
    max_pages = max(-(-(n + extra_tokens) // page) for n in lens) + 1
    num_pages = sum(-(-(n + extra_tokens) // page) for n in lens) + spare_pages
    cache = PagedKVCache(num_layers, B, HQ, HKV, D, page, max_pages, num_pages, case.dtype)
    return cache


def fill_and_step(cache, case, layer=0):
    """Prefill tokens [0, T_b - 1), start a decode step, append token T_b - 1."""
    lens = case.lengths
    B = len(lens)
    cache.seq_reset([max(n - 1, 0) for n in lens], reserve_tokens=0)
    k = to_dev(case.K, case.dtype)
    v = to_dev(case.V, case.dtype)
    cache.kv_prefill(layer, k, v)
    cache.step_begin()
    kn = torch.stack([k[b, :, max(lens[b] - 1, 0)] for b in range(B)]).contiguous()
    vn = torch.stack([v[b, :, max(lens[b] - 1, 0)] for b in range(B)]).contiguous()
    cache.kv_append(layer, kn, vn)
    return to_dev(case.q, case.dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, tol, what=""):
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3g} > {tol}"
    return err


def band_ok(S_row, j, k_top, recency):
    """Whether candidate page j lies in the selection boundary band of one row."""
    NP = len(S_row)
    NC = max(0, NP - recency)
    kk = min(k_top, NC)
    if kk == 0 or kk == NC:
        return False
    cand = np.sort(np.asarray(S_row[:NC]))[::-1]
    sk = cand[kk - 1]
    if sk < F32_MIN_NORMAL:
        return S_row[j] < F32_MIN_NORMAL or abs(S_row[j] - sk) <= BAND * max(sk, F32_MIN_NORMAL)
    return abs(S_row[j] - sk) <= BAND * sk


def check_selection(sel_row, count, S_row, k_top, recency, cap):
    """GPU selection vs the oracle's: exact except pages in the boundary band."""
    NP = len(S_row)
    ref = oracle.select_pages(S_row, k_top, recency)
    got = [int(x) for x in sel_row[:count]]
    assert count == len(ref) == min(NP, k_top + recency), (count, len(ref))
    assert got == sorted(set(got)), "selection not ascending / unique"
    assert all(int(x) == -1 for x in sel_row[count:cap]), "padding not -1"
    assert set(range(max(0, NP - recency), NP)) <= set(got), "recency window missing"
    for j in set(got) ^ set(ref):
        assert band_ok(S_row, j, k_top, recency), f"page {j} differs outside the band"
    return len(set(got) ^ set(ref))
