"""Planted mistakes in the oracle (CPU only): every one must be caught by a pin.

Each test swaps one oracle function for a plausibly wrong variant and checks that a
pin from the other oracle test files then fails.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.delta as odel
from tests import test_oracle_attention as TA
from tests import test_oracle_delta as TD
from tests import test_oracle_stack as TS


def _full_wrong_head_map(q, K, V, sm_scale):
    hq = q.shape[0]
    hkv = K.shape[0]
    out, lse, p = np.zeros_like(q), np.zeros(hq), np.zeros((hq, K.shape[1]))
    for h in range(hq):
        g = h % hkv  # interleaved instead of consecutive head groups
        out[h], lse[h], p[h], _ = oatt.attention_over_tokens(q[h], K[g], V[g], sm_scale)
    return out, lse, p


def test_mutant_head_map_caught(monkeypatch):
    monkeypatch.setattr(oracle, "full_attention", _full_wrong_head_map)
    with pytest.raises(AssertionError):
        TA.test_full_matches_torch_sdpa(8, 2, 64, 16, 1.0)


def test_mutant_dropped_scale_caught(monkeypatch):
    real = oatt.full_attention
    monkeypatch.setattr(oracle, "full_attention", lambda q, K, V, s: real(q, K, V, 1.0))
    with pytest.raises(AssertionError):
        TA.test_full_matches_torch_sdpa(28, 4, 333, 128, 128 ** -0.5)


def test_mutant_unnormalised_sparse_caught(monkeypatch):
    real_full = oatt.full_attention

    def sparse_no_renorm(q, K, V, sel, page, sm_scale):
        # weights taken from the full softmax and simply restricted to the selection
        _, _, p = real_full(q, K, V, sm_scale)
        hq, hkv, T = q.shape[0], K.shape[0], K.shape[1]
        G = hq // hkv
        if np.isscalar(sel[0]):
            sel = [sel] * hkv
        out, lse = np.zeros_like(q), np.zeros(hq)
        for h in range(hq):
            toks = oatt.selected_tokens(sel[h // G], T, page)
            out[h] = p[h, toks] @ V[h // G][toks]
        return out, lse

    monkeypatch.setattr(oracle, "sparse_attention", sparse_no_renorm)
    with pytest.raises(AssertionError):
        TA.test_sparse_equals_sdpa_on_gathered_tokens()


def test_mutant_sum_instead_of_max_caught(monkeypatch):
    real = odel.token_scores
    monkeypatch.setattr(TD, "token_scores", lambda p, hkv, agg="max", scope="group": real(p, hkv, "sum", scope))
    with pytest.raises(AssertionError):
        TD.test_token_scores_hand_example()


def test_mutant_page_boundary_off_by_one_caught(monkeypatch):
    def shifted(a, page):
        R, T = a.shape
        NP = -(-T // page)
        S = np.zeros((R, NP))
        for r in range(R):
            for j in range(NP):
                S[r, j] = np.sum(a[r, j * page + 1: min((j + 1) * page + 1, T)])
        return S

    monkeypatch.setattr(TD, "page_scores", shifted)
    with pytest.raises(AssertionError):
        TD.test_page_score_special_cases()


def _select_high_index_ties(S_row, k_top, recency):
    NP = len(S_row)
    fr = max(0, NP - recency)
    ranked = sorted(range(fr), key=lambda j: (-S_row[j], -j))
    return sorted(list(range(fr, NP)) + ranked[:k_top])


def _select_no_recency(S_row, k_top, recency):
    NP = len(S_row)
    ranked = sorted(range(NP), key=lambda j: (-S_row[j], j))
    return sorted(ranked[: k_top + recency])


def test_mutant_tie_break_caught(monkeypatch):
    monkeypatch.setattr(TD, "select_pages", _select_high_index_ties)
    with pytest.raises(AssertionError):
        TD.test_select_all_equal_scores_take_lowest_indices()
    S = [0.5, 0.5, 0.5, 0.25, 0.1]
    assert _select_high_index_ties(S, 2, 1) != TD.brute_force_top(S, 2, 1)


def test_mutant_dropped_recency_caught(monkeypatch):
    monkeypatch.setattr(TD, "select_pages", _select_no_recency)
    with pytest.raises(AssertionError):
        TD.test_select_all_equal_scores_take_lowest_indices()


def test_mutant_stale_selection_caught(monkeypatch):
    # sparse layers wrongly reuse the first delta-layer's selection for the whole stack
    real = oracle.stack_step

    def stale(tiers, inputs, sm, page, k, L, agg="max", scope="group"):
        res = real(tiers, inputs, sm, page, k, L, agg, scope)
        first = next(r["sel"] for r in res if "sel" in r)
        for r in res:
            if "sel_used" in r:
                r["sel_used"] = first
        return res

    monkeypatch.setattr(oracle, "stack_step", stale)
    with pytest.raises(AssertionError):
        TS.test_sparse_layers_use_latest_delta_selection()


# ---- fp8 rows (oracle.quant) ----
import oracle.quant as oq  # noqa: E402
from tests import test_oracle_quant as TQ  # noqa: E402


def test_mutant_e4m3_bias_caught(monkeypatch):
    real = oq.e4m3_decode
    monkeypatch.setattr(oq, "e4m3_decode", lambda c: real(c) / 2.0)  # exponent bias 8 instead of 7
    with pytest.raises(AssertionError):
        TQ.test_decode_matches_torch_float8_e4m3fn()


def test_mutant_ties_away_caught(monkeypatch):
    pos = oq._POS

    def encode_ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        hi = np.clip(np.searchsorted(pos, a, side="left"), 0, len(pos) - 1)
        lo = np.clip(hi - 1, 0, len(pos) - 1)
        pick = np.where(np.abs(a - pos[lo]) < np.abs(pos[hi] - a), lo, hi)
        return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)

    monkeypatch.setattr(oq, "e4m3_encode", encode_ties_away)
    with pytest.raises(AssertionError):
        TQ.test_encode_matches_torch_rne_including_ties()


def test_mutant_wrong_scale_constant_caught(monkeypatch):
    real_encode = oq.e4m3_encode

    def quantize_240(x):  # the largest value of the other E4M3 variant
        x32 = np.asarray(x, dtype=np.float32)
        scale = (np.max(np.abs(x32), axis=-1) / np.float32(240)).astype(np.float32)
        safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
        return real_encode(np.clip(x32 / safe[..., None], -448, 448)), scale

    monkeypatch.setattr(oq, "quantize_rows", quantize_240)
    with pytest.raises(AssertionError):
        TQ.test_quantize_rows_exact_on_representable_rows()
