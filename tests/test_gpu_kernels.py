"""GPU parity of every kernel through the C ABI against the CPU oracle.

Sizes span several sub-tiles, splits and a ragged tail; inputs come from the seeded
generator (workload.cases) and are exact in the stored dtype, so the oracle sees
the same values as the device.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.delta import page_scores as o_page_scores, token_scores as o_token_scores
from tests.gpu_util import (TOL, LSE_TOL, assert_close, check_selection, fill_and_step, host, make_cache,
                            to_dev, tdtype)
from workload.cases import random_case, plant_salient

pytestmark = pytest.mark.gpu

# id, dtype, B, Hq, Hkv, D, P, lengths
CASES = [
    ("f32_g4_d64_t1024", "f32", 1, 8, 2, 64, 16, [1024]),
    ("bf16_g7_d128_t8192", "bf16", 1, 28, 4, 128, 16, [8192]),
    ("bf16_ragged_p16", "bf16", 6, 28, 4, 128, 16, [1, 15, 16, 17, 1000, 2049]),
    ("bf16_ragged_p32_g4", "bf16", 4, 32, 8, 128, 32, [31, 32, 33, 3000]),
    ("bf16_g1_d64", "bf16", 2, 4, 4, 64, 16, [100, 700]),
    ("bf16_g16_d128", "bf16", 2, 16, 1, 128, 16, [257, 1300]),
    ("f32_g8_d128_p32", "f32", 2, 8, 1, 128, 32, [65, 999]),
    ("bf16_p64_g4", "bf16", 2, 8, 2, 64, 64, [65, 1300]),
]
IDS = [c[0] for c in CASES]


def _case(spec, seed=11):
    name, dtype, B, HQ, HKV, D, P, lens = spec
    scale = 1.0 / np.sqrt(D)
    c = random_case(seed, B, HQ, HKV, D, lens, dtype)
    G = HQ // HKV
    for b in range(B):
        T = lens[b]
        if T > 64:
            plant_salient(c, b, 0, [T // 7, T // 3, T // 2], G)
    return c, P, float(scale)


SCORE_RTOL = {"max": 6e-4, "sum": 1e-4}


def _budget(T, P):
    NP = -(-T // P)
    return max(1, NP // 5), 2


@pytest.mark.parametrize("spec", CASES, ids=IDS)
def test_full_attention(spec):
    case, P, sm = _case(spec)
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    out, lse = cache.attn_full(0, q, sm)
    torch.cuda.synchronize()
    for b, T in enumerate(case.lengths):
        ref, ref_lse, _ = oracle.full_attention(case.q[b], case.K[b, :, :T], case.V[b, :, :T], sm)
        assert_close(host(out[b]), ref, TOL[case.dtype], f"out b={b}")
        assert_close(host(lse[b]), ref_lse, LSE_TOL[case.dtype], f"lse b={b}")


@pytest.mark.parametrize("agg", ["max", "sum"])
@pytest.mark.parametrize("scope", ["group", "all"])
@pytest.mark.parametrize("spec", CASES, ids=IDS)
def test_delta_select(spec, agg, scope):
    case, P, sm = _case(spec)
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    T0 = case.lengths[0]
    k_top, rec = _budget(max(case.lengths), P)
    B = len(case.lengths)
    R = cache.sel_rows(scope)
    scores = torch.full((B, R, cache.max_pages), -7.0, dtype=torch.float32, device="cuda")
    out_f, lse_f = cache.attn_full(0, q, sm)
    out, lse, sel, cnt = cache.attn_delta_select(0, q, sm, k_top, rec, agg, scope, page_scores=scores,
                                                 sel_capacity=k_top + rec + 3)
    torch.cuda.synchronize()
    # the delta-layer's attention output is the full-attention output, bit for bit
    assert torch.equal(out, out_f) and torch.equal(lse, lse_f)
    hkv = case.K.shape[1]
    for b, T in enumerate(case.lengths):
        r = oracle.delta_layer(case.q[b], case.K[b, :, :T], case.V[b, :, :T], sm, P, k_top, rec, agg, scope)
        NP = -(-T // P)
        S = r["page_scores"]
        got = scores[b].cpu().numpy().astype(np.float64)
        # MAX scores come from fp16 weights relative to each (head, sub-tile) maximum:
        # relative error <= 2^-11; SUM scores from exact (max, sum) pairs
        np.testing.assert_allclose(got[:, :NP], S, rtol=SCORE_RTOL[agg], atol=1e-7)
        assert np.all(got[:, NP:] == -7.0)  # entries past NP untouched
        for row in range(R):
            check_selection(sel[b, row].cpu().numpy(), int(cnt[b, row]), S[row], k_top, rec, sel.shape[-1])


@pytest.mark.parametrize("spec", CASES, ids=IDS)
def test_sparse_attention(spec):
    case, P, sm = _case(spec)
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    k_top, rec = _budget(max(case.lengths), P)
    _, _, sel, cnt = cache.attn_delta_select(0, q, sm, k_top, rec)
    out, lse = cache.attn_sparse(0, q, sm, sel, cnt)
    torch.cuda.synchronize()
    hkv = case.K.shape[1]
    for b, T in enumerate(case.lengths):
        sels = [sel[b, g, :int(cnt[b, g])].cpu().tolist() for g in range(hkv)]  # the GPU's own selection
        ref, ref_lse = oracle.sparse_attention(case.q[b], case.K[b, :, :T], case.V[b, :, :T], sels, P, sm)
        assert_close(host(out[b]), ref, TOL[case.dtype], f"sparse out b={b}")
        assert_close(host(lse[b]), ref_lse, LSE_TOL[case.dtype], f"sparse lse b={b}")


@pytest.mark.parametrize("spec", CASES[:4], ids=IDS[:4])
def test_sparse_with_whole_context_equals_full(spec):
    case, P, sm = _case(spec)
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    NPmax = -(-max(case.lengths) // P)
    out_f, lse_f = cache.attn_full(0, q, sm)
    # budget covering the context: every page is selected
    _, _, sel, cnt = cache.attn_delta_select(0, q, sm, NPmax, 1)
    out_s, lse_s = cache.attn_sparse(0, q, sm, sel, cnt)
    torch.cuda.synchronize()
    for b, T in enumerate(case.lengths):
        NP = -(-T // P)
        assert int(cnt[b, 0]) == NP and sel[b, 0, :NP].cpu().tolist() == list(range(NP))
    assert_close(host(out_s), host(out_f), 1e-6 if case.dtype == "f32" else 8e-3, "sparse(all) vs full")
    assert_close(host(lse_s), host(lse_f), 1e-5, "lse")


def _tie_scores(rng, B, R, NP, levels):
    return (rng.integers(0, levels, size=(B, R, NP)) / levels).astype(np.float32)


# rows up to 8192 pages take the one-wave selector (16, 32, 64 or 128 keys per lane),
# longer ones the workgroup selector (keys staged in LDS up to 12288 pages, else global)
@pytest.mark.parametrize("NP,k_top,rec,levels", [
    (64, 8, 4, 5), (512, 96, 32, 3), (4100, 192, 64, 50), (1000, 0, 8, 4), (30, 40, 4, 3),
    (7, 3, 9, 2), (2049, 2048, 0, 2), (300, 17, 0, 1000000), (13000, 500, 16, 7), (1500, 100, 10, 3),
    (3000, 250, 40, 1000000), (8192, 700, 64, 11), (8193, 300, 20, 9)])
def test_page_select_on_oracle_scores_is_exact(NP, k_top, rec, levels):
    from layer_aware_kv_amd import PagedKVCache
    B, R, P = 3, 2, 16
    rng = np.random.default_rng(NP + k_top)
    S = _tie_scores(rng, B, R, NP, levels)
    S[0, 0, :] = 0.0  # an all-zero row
    cache = PagedKVCache(1, B, 2 * R, R, 64, P, NP + 1, B * (NP + 1), "bf16")
    lens = [NP * P, NP * P - 5, max(1, (NP // 2) * P)]
    cache.seq_reset(lens)
    dev = torch.zeros((B, R, NP + 1), dtype=torch.float32, device="cuda")
    dev[:, :, :NP] = torch.from_numpy(S).cuda()
    sel, cnt = cache.page_select(dev, k_top, rec)
    torch.cuda.synchronize()
    for b in range(B):
        np_b = -(-lens[b] // P)
        for r in range(R):
            row = S[b, r, :np_b]
            NC = max(0, np_b - rec)
            order = sorted(range(NC), key=lambda j: (-float(row[j]), j))[:k_top]  # float32 values
            ref = sorted(order + list(range(NC, np_b)))
            n = int(cnt[b, r])
            assert n == len(ref)
            assert sel[b, r, :n].cpu().tolist() == ref
            assert (sel[b, r, n:] == -1).all()


def test_page_select_special_values():
    """Scores that are NaN, negative, -0 or -inf order as 0; +inf is the largest; ties among
    them (and with real zeros) go to the lower page index."""
    from layer_aware_kv_amd import PagedKVCache
    B, R, P, NP = 2, 2, 16, 700
    rng = np.random.default_rng(5)
    S = rng.random((B, R, NP)).astype(np.float32) * 1e-3
    S[:, :, rng.choice(NP, 200, replace=False)] = 0.0
    S[0, 0, rng.choice(NP, 60, replace=False)] = np.nan
    S[0, 1, rng.choice(NP, 60, replace=False)] = -1.0
    S[1, 0, rng.choice(NP, 40, replace=False)] = -np.inf
    S[1, 0, rng.choice(NP, 5, replace=False)] = np.inf
    S[1, 1, rng.choice(NP, 50, replace=False)] = -0.0
    cache = PagedKVCache(1, B, 2 * R, R, 64, P, NP + 1, B * (NP + 1), "bf16")
    cache.seq_reset([NP * P] * B)
    dev = torch.zeros((B, R, NP + 1), dtype=torch.float32, device="cuda")
    dev[:, :, :NP] = torch.from_numpy(S).cuda()
    for k_top, rec in [(300, 10), (600, 20), (5, 0)]:
        sel, cnt = cache.page_select(dev, k_top, rec)
        torch.cuda.synchronize()
        for b in range(B):
            for r in range(R):
                row = [float(x) if (x > 0) else 0.0 for x in S[b, r]]  # NaN > 0 is False
                NC = NP - rec
                order = sorted(range(NC), key=lambda j: (-row[j], j))[:k_top]
                ref = sorted(order + list(range(NC, NP)))
                n = int(cnt[b, r])
                assert n == len(ref) and sel[b, r, :n].cpu().tolist() == ref, (b, r, k_top, rec)


@pytest.mark.parametrize("dtype,D,P", [("bf16", 128, 16), ("f32", 64, 16), ("bf16", 128, 32), ("bf16", 64, 64)])
def test_kv_prefill_append_gather_roundtrip(dtype, D, P):
    lens = [1, 17, 63, 200]
    case = random_case(5, 4, 4, 2, D, lens, dtype)
    cache = make_cache(case, P, num_layers=2, extra_tokens=40)
    cache.seq_reset([n - 1 for n in lens], reserve_tokens=0)
    k, v = to_dev(case.K, dtype), to_dev(case.V, dtype)
    cache.kv_prefill(1, k, v)
    # decode steps across page boundaries
    extra = random_case(6, 4, 4, 2, D, [40] * 4, dtype)
    kx, vx = to_dev(extra.K, dtype), to_dev(extra.V, dtype)
    for s in range(40):
        cache.step_begin()
        if s == 0:
            kn = torch.stack([k[b, :, lens[b] - 1] for b in range(4)]).contiguous()
            vn = torch.stack([v[b, :, lens[b] - 1] for b in range(4)]).contiguous()
        else:
            kn, vn = kx[:, :, s].contiguous(), vx[:, :, s].contiguous()
        cache.kv_append(1, kn, vn)
    assert cache.seq_lens_host() == [n + 39 for n in lens]
    assert cache.seq_lens.cpu().tolist()[:4] == [n + 39 for n in lens]
    for b in range(4):
        pt = cache.page_table_host(b)
        assert cache.page_table[b, :len(pt)].cpu().tolist() == pt
        for g in range(2):
            kg, vg = cache.kv_gather(1, b, g, 0, lens[b] + 39)
            exp_k = torch.cat([k[b, g, :lens[b]], kx[b, g, 1:40]])
            exp_v = torch.cat([v[b, g, :lens[b]], vx[b, g, 1:40]])
            assert torch.equal(kg, exp_k) and torch.equal(vg, exp_v)
    # single-row overwrite
    rows = torch.tensor([[0, 1, 0], [3, 0, 150], [2, 1, 10 ** 6]], dtype=torch.int32, device="cuda")
    kr = torch.randn(3, D, device="cuda").to(tdtype(dtype))
    cache.kv_write_rows(1, rows, kr)
    kg, _ = cache.kv_gather(1, 3, 0, 150, 1)
    assert torch.equal(kg[0], kr[1])
    kg, _ = cache.kv_gather(1, 0, 1, 0, 1)
    assert torch.equal(kg[0], kr[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("agg", ["max", "sum"])
def test_delta_and_sparse_wide_logit_range(dtype, agg):
    """Logits spread over about +-150 log2 units (q scaled by 32): many sub-tiles peak more
    than 64 log2 units below the running maximum, so the delta kernel takes their weights
    from the logits directly rather than from the probabilities, and the page scores of
    most pages underflow float32 (scored as tied at 0 by the selection band)."""
    B, HQ, HKV, D, P = 2, 28, 4, 128, 16
    case = random_case(31, B, HQ, HKV, D, [1500, 777], dtype, q_scale=32.0)
    sm = float(1.0 / np.sqrt(D))
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    k_top, rec = 20, 2
    scores = torch.full((B, HKV, cache.max_pages), -7.0, dtype=torch.float32, device="cuda")
    out, lse, sel, cnt = cache.attn_delta_select(0, q, sm, k_top, rec, agg, "group", page_scores=scores)
    out_s, lse_s = cache.attn_sparse(0, q, sm, sel, cnt)
    torch.cuda.synchronize()
    for b, T in enumerate(case.lengths):
        K, V = case.K[b, :, :T], case.V[b, :, :T]
        r = oracle.delta_layer(case.q[b], K, V, sm, P, k_top, rec, agg, "group")
        assert_close(host(out[b]), r["out"], TOL[dtype], f"out b={b}")
        assert_close(host(lse[b]), r["lse"], LSE_TOL[dtype], f"lse b={b}")
        NP = -(-T // P)
        np.testing.assert_allclose(scores[b].cpu().numpy().astype(np.float64)[:, :NP], r["page_scores"],
                                   rtol=SCORE_RTOL[agg], atol=1e-7)
        for g in range(HKV):
            check_selection(sel[b, g].cpu().numpy(), int(cnt[b, g]), r["page_scores"][g], k_top, rec,
                            sel.shape[-1])
        sels = [sel[b, g, :int(cnt[b, g])].cpu().tolist() for g in range(HKV)]
        ref, ref_lse = oracle.sparse_attention(case.q[b], K, V, sels, P, sm)
        assert_close(host(out_s[b]), ref, TOL[dtype], f"sparse b={b}")
        assert_close(host(lse_s[b]), ref_lse, LSE_TOL[dtype], f"sparse lse b={b}")


def test_edge_cases_empty_and_degenerate():
    from layer_aware_kv_amd import PagedKVCache
    # a sequence of length 0 (no decode step yet): out = 0, lse = -inf
    cache = PagedKVCache(1, 2, 8, 2, 64, 16, 8, 16, "bf16")
    cache.seq_reset([0, 20])
    case = random_case(3, 2, 8, 2, 64, [1, 20], "bf16")
    cache.kv_prefill(0, to_dev(case.K, "bf16"), to_dev(case.V, "bf16"))
    q = to_dev(case.q, "bf16")
    out, lse = cache.attn_full(0, q, 0.125)
    _, _, sel, cnt = cache.attn_delta_select(0, q, 0.125, 1, 1)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert cnt[0].tolist() == [0, 0] and (sel[0] == -1).all()
    ref, _, _ = oracle.full_attention(case.q[1], case.K[1, :, :20], case.V[1, :, :20], 0.125)
    assert_close(host(out[1]), ref, 2e-2)
    # k_top = 0 and recency = 0: an empty selection; sparse over it gives 0 / -inf
    _, _, sel, cnt = cache.attn_delta_select(0, q, 0.125, 0, 0, sel_capacity=1)
    out_s, lse_s = cache.attn_sparse(0, q, 0.125, sel, cnt)
    torch.cuda.synchronize()
    assert (cnt == 0).all() and torch.all(out_s == 0) and torch.all(torch.isneginf(lse_s))
    # an empty batch is a no-op
    cache.seq_reset([])
    e = torch.empty((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    cache.attn_full(0, e, 0.125, out=e, lse=torch.empty((0, 8), device="cuda"))
    torch.cuda.synchronize()


def test_invalid_selection_entries_are_skipped():
    case = random_case(9, 1, 8, 2, 64, [500], "bf16")
    cache = make_cache(case, 16)
    q = fill_and_step(cache, case)
    sel = torch.tensor([[[3, -1, 31, 999, 5], [0, 1, 2, -5, 40]]], dtype=torch.int32, device="cuda")
    cnt = torch.tensor([[5, 4]], dtype=torch.int32, device="cuda")
    out, _ = cache.attn_sparse(0, q, 0.125, sel, cnt)
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_attention(case.q[0], case.K[0, :, :500], case.V[0, :, :500], [[3, 31, 5], [0, 1, 2]],
                                     16, 0.125)
    assert_close(host(out[0]), ref, 2e-2)


def test_errors_reported_before_launch():
    from layer_aware_kv_amd import LakError
    case = random_case(9, 1, 8, 2, 64, [100], "bf16")
    cache = make_cache(case, 16)
    q = fill_and_step(cache, case)
    with pytest.raises(LakError, match="LAK_EINVAL"):
        cache.attn_delta_select(0, q, 0.125, 10, 10, sel_capacity=5)
    with pytest.raises(LakError, match="LAK_EINVAL"):
        cache.attn_full(3, q, 0.125)
    with pytest.raises(LakError, match="LAK_EINVAL"):
        cache.attn_delta_select(0, q, 0.125, -1, 1)


def test_deterministic_bitwise():
    spec = CASES[2]
    res = []
    for _ in range(2):
        case, P, sm = _case(spec)
        cache = make_cache(case, P)
        q = fill_and_step(cache, case)
        scores = torch.zeros((len(case.lengths), 4, cache.max_pages), device="cuda")
        out, lse, sel, cnt = cache.attn_delta_select(0, q, sm, 20, 3, page_scores=scores)
        out_s, lse_s = cache.attn_sparse(0, q, sm, sel, cnt)
        torch.cuda.synchronize()
        res.append([t.clone() for t in (out, lse, sel, cnt, scores, out_s, lse_s)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


FUSE_CASES = [CASES[0], CASES[2], CASES[3], CASES[6]]


@pytest.mark.parametrize("spec", FUSE_CASES, ids=[c[0] for c in FUSE_CASES])
def test_fused_append_matches_separate_append(spec):
    """An attention call given k_new / v_new equals kv_append followed by the call."""
    case, P, sm = _case(spec)
    B = len(case.lengths)
    cache_a = make_cache(case, P)
    q = fill_and_step(cache_a, case)
    k_top, rec = _budget(max(case.lengths), P)
    out_f, lse_f = cache_a.attn_full(0, q, sm)
    out_d, lse_d, sel, cnt = cache_a.attn_delta_select(0, q, sm, k_top, rec)
    out_s, lse_s = cache_a.attn_sparse(0, q, sm, sel, cnt)
    k, v = to_dev(case.K, case.dtype), to_dev(case.V, case.dtype)
    kn = torch.stack([k[b, :, case.lengths[b] - 1] for b in range(B)]).contiguous()
    vn = torch.stack([v[b, :, case.lengths[b] - 1] for b in range(B)]).contiguous()
    for tier in ("full", "delta", "sparse"):
        cache_b = make_cache(case, P)
        cache_b.seq_reset([n - 1 for n in case.lengths])
        cache_b.kv_prefill(0, k, v)
        cache_b.step_begin()
        if tier == "full":
            o, l = cache_b.attn_full(0, q, sm, k_new=kn, v_new=vn)
            ref = (out_f, lse_f)
        elif tier == "delta":
            o, l, s2, c2 = cache_b.attn_delta_select(0, q, sm, k_top, rec, k_new=kn, v_new=vn)
            ref = (out_d, lse_d)
        else:
            o, l = cache_b.attn_sparse(0, q, sm, sel, cnt, k_new=kn, v_new=vn)
            ref = (out_s, lse_s)
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), tier
        if tier == "delta":
            assert torch.equal(s2, sel) and torch.equal(c2, cnt)
        for b in range(B):
            for g in range(case.K.shape[1]):
                kg, vg = cache_b.kv_gather(0, b, g, case.lengths[b] - 1, 1)
                assert torch.equal(kg[0], kn[b, g]) and torch.equal(vg[0], vn[b, g])


def test_fidelity_recall_matches_oracle_mass():
    """The device recall exp(lse_sparse - lse_full) equals the oracle's full-softmax
    mass of the selected tokens."""
    from layer_aware_kv_amd import fidelity
    from oracle.attention import selected_tokens
    case, P, sm = _case(CASES[2])
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    out_f, lse_f = cache.attn_full(0, q, sm)
    _, _, sel, cnt = cache.attn_delta_select(0, q, sm, 12, 2)
    _, lse_s = cache.attn_sparse(0, q, sm, sel, cnt)
    rec = fidelity.selection_recall(lse_s, lse_f).cpu().numpy()
    G = case.q.shape[1] // case.K.shape[1]
    for b, T in enumerate(case.lengths):
        _, _, p = oracle.full_attention(case.q[b], case.K[b, :, :T], case.V[b, :, :T], sm)
        for h in range(case.q.shape[1]):
            toks = selected_tokens(sel[b, h // G, :int(cnt[b, h // G])].cpu().tolist(), T, P)
            assert abs(rec[b, h] - p[h, toks].sum()) < 5e-3


@pytest.mark.parametrize("kv", ["bf16", "f32", "fp8"])
def test_fused_append_sparse_without_the_token_page(kv):
    """A sparse call given k_new / v_new whose selection leaves out the page of this
    step's token still appends it (split 0's store) and attends only to the selection."""
    from layer_aware_kv_amd import PagedKVCache
    from oracle import quant as Q
    act = "bf16" if kv == "fp8" else kv
    lens = [300, 129]
    case = random_case(31, 2, 8, 2, 64, lens, act)
    out, kg = {}, {}
    for fused in (True, False):
        cache = PagedKVCache(1, 2, 8, 2, 64, 16, 24, 48, kv)
        cache.seq_reset([n - 1 for n in lens])
        k, v = to_dev(case.K, act), to_dev(case.V, act)
        cache.kv_prefill(0, k, v)
        cache.step_begin()
        kn = torch.stack([k[b, :, lens[b] - 1] for b in range(2)]).contiguous()
        vn = torch.stack([v[b, :, lens[b] - 1] for b in range(2)]).contiguous()
        q = to_dev(case.q, act)
        sel = torch.tensor([[[0, 3, 5, -1], [1, 2, 7, -1]], [[0, 2, -1, -1], [4, 5, 6, -1]]], dtype=torch.int32,
                           device="cuda")
        cnt = torch.tensor([[3, 3], [2, 3]], dtype=torch.int32, device="cuda")
        if fused:
            o, _ = cache.attn_sparse(0, q, 0.125, sel, cnt, k_new=kn, v_new=vn)
        else:
            cache.kv_append(0, kn, vn)
            o, _ = cache.attn_sparse(0, q, 0.125, sel, cnt)
        torch.cuda.synchronize()
        out[fused] = o.clone()
        kg[fused] = [cache.kv_gather(0, b, g, lens[b] - 1, 1) for b in range(2) for g in range(2)]
    assert torch.equal(out[True], out[False])
    for (k1, v1), (k2, v2) in zip(kg[True], kg[False]):
        assert torch.equal(k1, k2) and torch.equal(v1, v2)
    for b, T in enumerate(lens):
        K, V = case.K[b, :, :T], case.V[b, :, :T]
        if kv == "fp8":
            K, V = Q.quantize_dequantize(K), Q.quantize_dequantize(V)
        sels = [[j for j in sel[b, g, :int(cnt[b, g])].tolist()] for g in range(2)]
        ref, _ = oracle.sparse_attention(case.q[b], K, V, sels, 16, 0.125)
        assert_close(host(out[True][b]), ref, TOL["f32" if kv == "f32" else "bf16"], f"b={b}")


def test_attention_calls_replay_in_a_graph():
    """The attention entry points launch kernels only (no memset, no host wait), so a
    captured full / delta-select / sparse sequence replays exactly: every replay,
    separated by eager work and synchronisation, equals the eager result."""
    case, P, sm = _case(CASES[2])
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    out_f, lse_f = cache.attn_full(0, q, sm)
    out_d, lse_d, sel, cnt = cache.attn_delta_select(0, q, sm, 20, 3)
    out_s, lse_s = cache.attn_sparse(0, q, sm, sel, cnt)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out_f, lse_f, out_d, lse_d, sel, cnt, out_s, lse_s)]
    bufs = [torch.empty_like(t) for t in ref]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        cache.attn_full(0, q, sm, bufs[0], bufs[1])
        cache.attn_delta_select(0, q, sm, 20, 3, out=bufs[2], lse=bufs[3], sel=bufs[4], sel_count=bufs[5])
        cache.attn_sparse(0, q, sm, bufs[4], bufs[5], out=bufs[6], lse=bufs[7])
    for rep in range(3):
        for b in bufs:
            b.zero_()
        cache.attn_full(0, q, 0.5 * sm)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp in zip(bufs, ref):
            assert torch.equal(got, exp), f"replay {rep}"
