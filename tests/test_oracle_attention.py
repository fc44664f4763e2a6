"""Pins for oracle.attention against library routines, closed forms and invariants."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _rand(rng, hq, hkv, T, D, scale=1.0):
    q = rng.standard_normal((hq, D)) * scale
    K = rng.standard_normal((hkv, T, D))
    V = rng.standard_normal((hkv, T, D))
    return q, K, V


def _sdpa(q, K, V, sm_scale, G):
    """torch's scaled_dot_product_attention on CPU in float64; GQA by repeat_interleave."""
    qt = torch.from_numpy(q)[None, :, None, :]
    Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]
    Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=sm_scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,T,D,scale", [
    (8, 2, 1024, 64, 1.0), (28, 4, 333, 128, 128 ** -0.5), (4, 4, 17, 32, 0.3), (7, 1, 1, 16, 1.0),
    (32, 8, 100, 128, 128 ** -0.5)])
def test_full_matches_torch_sdpa(hq, hkv, T, D, scale):
    rng = np.random.default_rng(hq * 1000 + T)
    q, K, V = _rand(rng, hq, hkv, T, D)
    out, lse, p = oracle.full_attention(q, K, V, scale)
    ref = _sdpa(q, K, V, scale, hq // hkv)
    assert np.max(np.abs(out - ref)) < 1e-12
    # LSE against scipy's logsumexp of the scaled logits, per head with g = h // G
    G = hq // hkv
    for h in range(hq):
        s = scale * K[h // G] @ q[h]
        assert abs(lse[h] - logsumexp(s)) < 1e-12
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    assert np.all(p >= 0)


def test_full_closed_forms():
    rng = np.random.default_rng(3)
    hq, hkv, T, D = 6, 2, 50, 16
    q = rng.standard_normal((hq, D))
    # identical keys -> uniform weights -> output is the mean of V, lse = s + ln T
    K = np.broadcast_to(rng.standard_normal(D), (hkv, T, D)).copy()
    V = rng.standard_normal((hkv, T, D))
    out, lse, p = oracle.full_attention(q, K, V, 0.5)
    for h in range(hq):
        g = h // 3
        assert np.allclose(out[h], V[g].mean(axis=0), atol=1e-13)
        assert abs(lse[h] - (0.5 * K[g, 0] @ q[h] + np.log(T))) < 1e-12
        assert np.allclose(p[h], 1.0 / T)
    # constant V -> output is that constant
    K = rng.standard_normal((hkv, T, D))
    V = np.broadcast_to(rng.standard_normal(D), (hkv, T, D)).copy()
    out, _, _ = oracle.full_attention(q, K, V, 1.0)
    assert np.allclose(out, V[0, 0][None, :], atol=1e-13)
    # one dominant key -> output is that key's value
    K = rng.standard_normal((hkv, T, D)) * 0.01
    K[:, 17] = q[0] * 100.0
    V = rng.standard_normal((hkv, T, D))
    out, _, p = oracle.full_attention(q[:1].repeat(hq, 0), K, V, 1.0)
    assert np.allclose(out[0], V[0, 17], atol=1e-9)
    # single token: weight 1, lse = its logit
    out, lse, p = oracle.full_attention(q, K[:, :1], V[:, :1], 0.7)
    assert np.allclose(out, np.repeat(V[:, 0], 3, axis=0)) and np.allclose(p, 1.0)
    assert np.allclose(lse, [0.7 * K[h // 3, 0] @ q[h] for h in range(hq)])


@pytest.mark.parametrize("T,page", [(1024, 16), (1000, 16), (77, 32), (5, 16)])
def test_sparse_all_pages_equals_full(T, page):
    rng = np.random.default_rng(T)
    q, K, V = _rand(rng, 8, 2, T, 64)
    NP = -(-T // page)
    out_f, lse_f, _ = oracle.full_attention(q, K, V, 0.125)
    out_s, lse_s = oracle.sparse_attention(q, K, V, [list(range(NP))] * 2, page, 0.125)
    assert np.max(np.abs(out_f - out_s)) < 1e-13 and np.max(np.abs(lse_f - lse_s)) < 1e-12


def test_sparse_equals_sdpa_on_gathered_tokens():
    rng = np.random.default_rng(11)
    hq, hkv, T, D, page = 8, 2, 203, 32, 16  # 13 pages, the last one partial (11 tokens)
    q, K, V = _rand(rng, hq, hkv, T, D)
    sel = [[0, 3, 4, 9, 12], [1, 2, 12]]
    out, lse = oracle.sparse_attention(q, K, V, sel, page, 0.2)
    for g in range(hkv):
        toks = [t for j in sel[g] for t in range(j * page, min((j + 1) * page, T))]
        assert len(toks) == (len(sel[g]) - 1) * page + 11
        heads = slice(g * 4, (g + 1) * 4)
        ref = _sdpa(q[heads], K[g:g + 1, toks], V[g:g + 1, toks], 0.2, 4)
        assert np.max(np.abs(out[heads] - ref)) < 1e-12
        for h in range(g * 4, (g + 1) * 4):
            assert abs(lse[h] - logsumexp(0.2 * K[g, toks] @ q[h])) < 1e-12
    # a single shared list is used for every KV head
    out1, _ = oracle.sparse_attention(q, K, V, [0, 5], page, 0.2)
    out2, _ = oracle.sparse_attention(q, K, V, [[0, 5], [0, 5]], page, 0.2)
    assert np.array_equal(out1, out2)


def test_selected_tokens_masks_partial_page():
    from oracle.attention import selected_tokens
    assert selected_tokens([0, 2], 40, 16).tolist() == list(range(16)) + list(range(32, 40))
    assert selected_tokens([], 40, 16).size == 0


def test_selection_mass_identity():
    """Attention mass of the selected tokens under the full softmax equals
    exp(lse_sparse - lse_full): the recall measure of the fidelity study."""
    rng = np.random.default_rng(21)
    hq, hkv, T, D, page = 8, 2, 300, 32, 16
    q, K, V = _rand(rng, hq, hkv, T, D)
    sel = [[0, 4, 7, 18], [2, 3, 18]]
    _, lse_f, p = oracle.full_attention(q, K, V, 0.3)
    _, lse_s = oracle.sparse_attention(q, K, V, sel, page, 0.3)
    from oracle.attention import selected_tokens
    for h in range(hq):
        toks = selected_tokens(sel[h // 4], T, page)
        assert abs(p[h, toks].sum() - np.exp(lse_s[h] - lse_f[h])) < 1e-12
