"""Pins for the oracle's stack step: the pages' schedule facts and stated invariants."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_tiers_from_pages_delta_lists():
    for model, n, lst in _golden_rows("pages_delta_layers.txt"):
        deltas = [int(x) for x in lst.split(",")]
        tiers = oracle.layer_tiers(int(n), [0, 1], deltas)
        assert tiers[0] == tiers[1] == "full"
        assert tiers[2] == "delta"          # the first delta-layer is layer 2 (Main Findings)
        assert [i for i, t in enumerate(tiers) if t == "delta"] == deltas
        assert tiers.count("sparse") == int(n) - 2 - len(deltas)


def _stack_inputs(rng, n_layers, hq, hkv, T, D):
    return [(rng.standard_normal((hq, D)) * 0.3, rng.standard_normal((hkv, T, D)),
             rng.standard_normal((hkv, T, D))) for _ in range(n_layers)]


def test_all_delta_stack_equals_all_full():
    # with every layer a delta-layer (or full), DELTA is full attention (Main Findings:
    # runtime tends to full attention's as the delta-layer count nears the layer count)
    rng = np.random.default_rng(1)
    inputs = _stack_inputs(rng, 6, 8, 2, 300, 32)
    full = oracle.stack_step(["full"] * 6, inputs, 1.0, 16, 2, 1)
    deltas = oracle.stack_step(["full", "full"] + ["delta"] * 4, inputs, 1.0, 16, 2, 1)
    for a, b in zip(full, deltas):
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


def test_budget_covering_context_equals_all_full():
    rng = np.random.default_rng(2)
    T, page = 250, 16  # 16 pages
    inputs = _stack_inputs(rng, 6, 8, 2, T, 32)
    tiers = oracle.layer_tiers(6, [0, 1], [2])
    full = oracle.stack_step(["full"] * 6, inputs, 1.0, page, 2, 1)
    for k, L in [(14, 2), (0, 16), (100, 0), (10, 10)]:
        res = oracle.stack_step(tiers, inputs, 1.0, page, k, L)
        for a, b in zip(full, res):
            assert np.max(np.abs(a["out"] - b["out"])) < 1e-13


def test_sparse_layers_use_latest_delta_selection():
    rng = np.random.default_rng(4)
    inputs = _stack_inputs(rng, 6, 8, 2, 400, 32)
    tiers = ["full", "full", "delta", "sparse", "delta", "sparse"]
    res = oracle.stack_step(tiers, inputs, 1.0, 16, 3, 2)
    assert res[3]["sel_used"] == res[2]["sel"]
    assert res[5]["sel_used"] == res[4]["sel"]
    # a small budget really changes the sparse output
    full5, _, _ = oracle.full_attention(*inputs[5], 1.0)
    assert np.max(np.abs(full5 - res[5]["out"])) > 1e-3


def test_sparse_before_delta_is_an_error():
    rng = np.random.default_rng(4)
    inputs = _stack_inputs(rng, 2, 4, 1, 20, 8)
    with pytest.raises(ValueError):
        oracle.stack_step(["full", "sparse"], inputs, 1.0, 16, 1, 1)


def test_no_eviction_dropped_page_can_return():
    # the full cache stays; a page unselected at one step is selectable at the next
    # ("Methodology in Plain English": no token is dropped from the KV cache)
    rng = np.random.default_rng(8)
    hq, hkv, T, D = 4, 1, 16 * 10, 16
    K = rng.standard_normal((hkv, T, D)) * 0.05
    V = rng.standard_normal((hkv, T, D))
    q1 = rng.standard_normal((hq, D))
    K[0, 2 * 16] = q1[0] * 3
    r1 = oracle.delta_layer(q1, K, V, 1.0, 16, 1, 1)
    q2 = -q1
    K2 = K.copy()
    K2[0, 5 * 16] = q2[0] * 3
    r2 = oracle.delta_layer(q2, K2, V, 1.0, 16, 1, 1)
    r3 = oracle.delta_layer(q1, K2, V, 1.0, 16, 1, 1)
    assert r1["sel"][0] == [2, 9] and r2["sel"][0] == [5, 9] and r3["sel"][0] == [2, 9]


def test_pages_budget_arithmetic():
    for K, P, L, bt, rt in _golden_rows("pages_budgets.txt"):
        K, P, L, bt, rt = map(int, (K, P, L, bt, rt))
        # the oracle's selection of K older pages plus L recent pages covers K*P + L*P tokens
        NP = 4 * (K + L)
        T = NP * P
        sel = oracle.select_pages(np.arange(NP, dtype=float)[::-1], K, L)
        from oracle.attention import selected_tokens
        toks = selected_tokens(sel, T, P)
        assert len(toks) == bt + rt and len([j for j in sel if j >= NP - L]) * P == rt
