"""Pins for the oracle's delta-layer scoring and selection (brute force, closed forms)."""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle.delta import page_scores, select_pages, token_scores


def test_token_scores_hand_example():
    # 4 heads, 2 KV groups (G = 2), 3 tokens; weights chosen by hand (rows sum to 1)
    p = np.array([[0.5, 0.25, 0.25],
                  [0.1, 0.6, 0.3],
                  [0.2, 0.2, 0.6],
                  [0.7, 0.1, 0.2]])
    assert np.allclose(token_scores(p, 2, "max"), [[0.5, 0.6, 0.3], [0.7, 0.2, 0.6]])
    assert np.allclose(token_scores(p, 2, "sum"), [[0.6, 0.85, 0.55], [0.9, 0.3, 0.8]])
    assert np.allclose(token_scores(p, 2, "max", scope="all"), [[0.7, 0.6, 0.6]])
    # pages of 2 tokens: [t0 t1] [t2]
    assert np.allclose(page_scores(token_scores(p, 2, "max"), 2), [[1.1, 0.3], [0.9, 0.6]])


def _softmax_rows(rng, hq, T):
    s = rng.standard_normal((hq, T)) * 3
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("hq,hkv,T,page", [(8, 2, 1024, 16), (28, 4, 1000, 16), (32, 8, 95, 32)])
def test_page_score_sum_invariants(hq, hkv, T, page):
    rng = np.random.default_rng(T)
    p = _softmax_rows(rng, hq, T)
    G = hq // hkv
    S_sum = page_scores(token_scores(p, hkv, "sum"), page)
    S_max = page_scores(token_scores(p, hkv, "max"), page)
    NP = -(-T // page)
    assert S_sum.shape == (hkv, NP)
    # SUM: each group's page scores add up to G (each head's weights sum to 1)
    assert np.allclose(S_sum.sum(axis=1), G, atol=1e-12)
    # MAX: between one head's mass and the group's mass
    tot = S_max.sum(axis=1)
    assert np.all(tot >= 1.0 - 1e-12) and np.all(tot <= G + 1e-12)
    assert np.all(S_max >= 0) and np.all(S_max <= S_sum + 1e-15)
    # scope "all" sums to Hq (SUM)
    assert np.allclose(page_scores(token_scores(p, hkv, "sum", "all"), page).sum(), hq)


def test_page_score_special_cases():
    rng = np.random.default_rng(5)
    p = _softmax_rows(rng, 4, 37)
    # G = 1: MAX and SUM agree
    assert np.allclose(page_scores(token_scores(p, 4, "max"), 16), page_scores(token_scores(p, 4, "sum"), 16))
    # P = 1: page scores are token scores
    a = token_scores(p, 2, "max")
    assert np.array_equal(page_scores(a, 1), a)
    # partial last page: 37 = 2*16 + 5 -> the last page sums 5 tokens
    S = page_scores(a, 16)
    assert np.allclose(S[:, 2], a[:, 32:37].sum(axis=1))


def brute_force_top(S, k, recency):
    """Every size-k subset of the older pages; the one of largest total score, and among
    equal totals the lexicographically smallest sorted tuple."""
    NP = len(S)
    first_recent = max(0, NP - recency)
    C = list(range(first_recent))
    kk = min(k, len(C))
    best_key, best = None, None
    for subset in itertools.combinations(C, kk):
        key = (-sum(S[j] for j in subset), subset)
        if best_key is None or key < best_key:
            best_key, best = key, subset
    return sorted(list(best) + list(range(first_recent, NP)))


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(0, 6), min_size=1, max_size=11), st.integers(0, 6), st.integers(0, 5))
def test_select_equals_brute_force(levels, k, recency):
    # small integer levels give many ties; scores are exact dyadic values
    S = [lv / 8.0 for lv in levels]
    assert select_pages(S, k, recency) == brute_force_top(S, k, recency)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(0, 1, allow_nan=False), min_size=1, max_size=40), st.integers(0, 45),
       st.integers(0, 45))
def test_select_invariants(S, k, recency):
    sel = select_pages(S, k, recency)
    NP = len(S)
    assert sel == sorted(set(sel))
    assert len(sel) == min(NP, k + recency)
    assert set(range(max(0, NP - recency), NP)) <= set(sel)
    # equals a stable argsort of -S over the older pages
    first_recent = max(0, NP - recency)
    order = np.argsort(-np.asarray(S[:first_recent]), kind="stable")[:k]
    assert sel == sorted(order.tolist() + list(range(first_recent, NP)))


def test_select_all_equal_scores_take_lowest_indices():
    assert select_pages([0.25] * 20, 5, 3) == [0, 1, 2, 3, 4, 17, 18, 19]
    assert select_pages([0.0] * 6, 10, 2) == list(range(6))
    assert select_pages([1.0, 2.0, 3.0], 0, 0) == []
    assert select_pages([3.0, 1.0, 2.0, 0.5], 2, 0) == [0, 2]


def test_delta_layer_selects_salient_pages():
    # plant strongly attended keys in pages 3 and 7 of group 0 and page 1 of group 1
    rng = np.random.default_rng(9)
    hq, hkv, T, D, page = 8, 2, 16 * 12, 32, 16
    q = rng.standard_normal((hq, D))
    K = rng.standard_normal((hkv, T, D)) * 0.1
    V = rng.standard_normal((hkv, T, D))
    K[0, 3 * 16 + 5] = q[0] * 2
    K[0, 7 * 16 + 2] = q[1] * 2
    K[1, 1 * 16 + 9] = q[5] * 2
    r = oracle.delta_layer(q, K, V, 1.0, page, k_top=2, recency=2, agg="max")
    assert r["sel"][0] == [3, 7, 10, 11]
    assert r["sel"][1][-2:] == [10, 11] and 1 in r["sel"][1]
    assert len(r["sel"]) == 2
    r_all = oracle.delta_layer(q, K, V, 1.0, page, k_top=3, recency=2, agg="max", scope="all")
    assert len(r_all["sel"]) == 1 and {1, 3, 7} <= set(r_all["sel"][0])
