"""GPU parity of fp8 (OCP E4M3, per-row scale) KV pages through the C ABI.

Rows go in as bfloat16; the device's codes and scales must equal the oracle's
encoding bit for bit, and every tier's attention must match the oracle run on
the dequantized rows (code * scale, float64) within the bfloat16 tolerances."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant as Q
from tests.gpu_util import LSE_TOL, TOL, assert_close, check_selection, host, to_dev
from workload.cases import plant_salient, random_case

pytestmark = pytest.mark.gpu

# id, B, Hq, Hkv, D, P, lengths
CASES = [
    ("fp8_g7_d128_t8192", 1, 28, 4, 128, 16, [8192]),
    ("fp8_ragged_p16", 6, 28, 4, 128, 16, [1, 15, 16, 17, 1000, 2049]),
    ("fp8_ragged_p32_g4", 4, 32, 8, 128, 32, [31, 32, 33, 3000]),
    ("fp8_g1_d64", 2, 4, 4, 64, 16, [100, 700]),
    ("fp8_g16_p64", 2, 16, 1, 128, 64, [257, 1300]),
]
IDS = [c[0] for c in CASES]


def _case(spec, seed=21):
    _, B, HQ, HKV, D, P, lens = spec
    c = random_case(seed, B, HQ, HKV, D, lens, "bf16")
    for b in range(B):
        if lens[b] > 64:
            plant_salient(c, b, 0, [lens[b] // 7, lens[b] // 3, lens[b] // 2], HQ // HKV)
    return c, P, float(1.0 / np.sqrt(D))


def _cache(case, P, layers=1, extra=1):
    from layer_aware_kv_amd import PagedKVCache
    B, HQ, D = case.q.shape
    HKV = case.K.shape[1]
    lens = case.lengths
    max_pages = max(-(-(n + extra) // P) for n in lens) + 1
    num_pages = sum(-(-(n + extra) // P) for n in lens) + 4
    return PagedKVCache(layers, B, HQ, HKV, D, P, max_pages, num_pages, "fp8")


def _fill(cache, case, layer=0):
    """Prefill tokens [0, T_b - 1), one decode step, append token T_b - 1 (bfloat16 rows)."""
    lens = case.lengths
    B = len(lens)
    cache.seq_reset([max(n - 1, 0) for n in lens])
    k, v = to_dev(case.K, "bf16"), to_dev(case.V, "bf16")
    cache.kv_prefill(layer, k, v)
    cache.step_begin()
    kn = torch.stack([k[b, :, max(lens[b] - 1, 0)] for b in range(B)]).contiguous()
    vn = torch.stack([v[b, :, max(lens[b] - 1, 0)] for b in range(B)]).contiguous()
    cache.kv_append(layer, kn, vn)
    return to_dev(case.q, "bf16"), kn, vn


def _dq(case, b, T):
    return Q.quantize_dequantize(case.K[b, :, :T]), Q.quantize_dequantize(case.V[b, :, :T])


def _check_codes(cache, case, layer=0):
    for b, T in enumerate(case.lengths):
        for g in range(case.K.shape[1]):
            kc, vc = cache.kv_gather(layer, b, g, 0, T)
            ks, vs = cache.kv_gather_scales(layer, b, g, 0, T)
            rk, rks = Q.quantize_rows(case.K[b, g, :T])
            rv, rvs = Q.quantize_rows(case.V[b, g, :T])
            assert np.array_equal(kc.cpu().numpy(), rk), f"K codes b={b} g={g}"
            assert np.array_equal(vc.cpu().numpy(), rv), f"V codes b={b} g={g}"
            assert np.array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32)), f"K scales b={b} g={g}"
            assert np.array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32)), f"V scales b={b} g={g}"


@pytest.mark.parametrize("spec", CASES, ids=IDS)
def test_fp8_codes_and_scales_bit_exact(spec):
    case, P, _ = _case(spec)
    cache = _cache(case, P)
    _fill(cache, case)
    torch.cuda.synchronize()
    _check_codes(cache, case)


@pytest.mark.parametrize("spec", CASES, ids=IDS)
def test_fp8_full_attention(spec):
    case, P, sm = _case(spec)
    cache = _cache(case, P)
    q, _, _ = _fill(cache, case)
    out, lse = cache.attn_full(0, q, sm)
    torch.cuda.synchronize()
    for b, T in enumerate(case.lengths):
        K, V = _dq(case, b, T)
        ref, ref_lse, _ = oracle.full_attention(case.q[b], K, V, sm)
        assert_close(host(out[b]), ref, TOL["bf16"], f"out b={b}")
        assert_close(host(lse[b]), ref_lse, LSE_TOL["bf16"], f"lse b={b}")


@pytest.mark.parametrize("agg,scope", [("max", "group"), ("sum", "group"), ("max", "all")])
@pytest.mark.parametrize("spec", CASES, ids=IDS)
def test_fp8_delta_select_and_sparse(spec, agg, scope):
    case, P, sm = _case(spec)
    cache = _cache(case, P)
    q, _, _ = _fill(cache, case)
    NPmax = -(-max(case.lengths) // P)
    k_top, rec = max(1, NPmax // 5), 2
    B = len(case.lengths)
    R = cache.sel_rows(scope)
    scores = torch.full((B, R, cache.max_pages), -7.0, dtype=torch.float32, device="cuda")
    out_f, lse_f = cache.attn_full(0, q, sm)
    out, lse, sel, cnt = cache.attn_delta_select(0, q, sm, k_top, rec, agg, scope, page_scores=scores)
    out_s, lse_s = cache.attn_sparse(0, q, sm, sel, cnt, scope)
    torch.cuda.synchronize()
    assert torch.equal(out, out_f) and torch.equal(lse, lse_f)
    hkv = case.K.shape[1]
    for b, T in enumerate(case.lengths):
        K, V = _dq(case, b, T)
        r = oracle.delta_layer(case.q[b], K, V, sm, P, k_top, rec, agg, scope)
        NP = -(-T // P)
        got = scores[b].cpu().numpy().astype(np.float64)
        # MAX: fp16 weights relative to each (head, sub-tile) maximum, relative error <= 2^-11
        np.testing.assert_allclose(got[:, :NP], r["page_scores"], rtol=6e-4 if agg == "max" else 1e-4, atol=1e-7)
        for row in range(R):
            check_selection(sel[b, row].cpu().numpy(), int(cnt[b, row]), r["page_scores"][row], k_top, rec,
                            sel.shape[-1])
        sels = [sel[b, (g if R > 1 else 0), :int(cnt[b, (g if R > 1 else 0)])].cpu().tolist() for g in range(hkv)]
        ref, ref_lse = oracle.sparse_attention(case.q[b], K, V, sels, P, sm)
        assert_close(host(out_s[b]), ref, TOL["bf16"], f"sparse out b={b}")
        assert_close(host(lse_s[b]), ref_lse, LSE_TOL["bf16"], f"sparse lse b={b}")


def test_fp8_every_code_decodes_exactly():
    """Rows that are 2^k times E4M3 values with a +-448 entry encode to exactly those
    codes (scale 2^k); together they hold all 254 finite codes, so attention over
    them checks the device's widening of every code against the format."""
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    B, HQ, HKV, D, P, T = 1, 8, 2, 128, 16, 96
    case = random_case(4, B, HQ, HKV, D, [T], "bf16")
    for kind in (case.K, case.V):
        codes = np.resize(rng.permutation(np.tile(finite, 2 * T * D // 254 + 1)), (HKV, T, D)).astype(np.uint8)
        codes[..., 5] = np.where(rng.random((HKV, T)) < 0.5, 0x7E, 0xFE)
        rows = Q.e4m3_decode(codes) * np.exp2(rng.integers(-12, 2, size=(HKV, T)))[..., None]
        kind[0] = rows
    cache = _cache(case, P)
    q, _, _ = _fill(cache, case)
    out, lse = cache.attn_full(0, q, 1.0 / 64)
    torch.cuda.synchronize()
    _check_codes(cache, case)
    assert np.array_equal(_dq(case, 0, T)[0], case.K[0])  # exact rows
    ref, ref_lse, _ = oracle.full_attention(case.q[0], case.K[0], case.V[0], 1.0 / 64)
    assert_close(host(out[0]), ref, 2e-2 * np.abs(ref).max(), "out")
    assert_close(host(lse[0]), ref_lse, LSE_TOL["bf16"], "lse")


def test_fp8_zero_rows_and_write_rows():
    case = random_case(8, 2, 8, 2, 64, [40, 300], "bf16")
    case.K[1, 0, 17] = 0.0
    case.V[1, 1, 200] = 0.0
    cache = _cache(case, 16, extra=2)
    q, _, _ = _fill(cache, case)
    torch.cuda.synchronize()
    _check_codes(cache, case)
    ks, vs = cache.kv_gather_scales(0, 1, 1, 200, 1)
    assert float(vs[0]) == 0.0
    # single-row overwrite re-encodes the K and V rows (the out-of-range third row is skipped)
    rows = torch.tensor([[1, 0, 17], [0, 1, 3], [1, 1, 10 ** 6]], dtype=torch.int32, device="cuda")
    new = random_case(9, 1, 8, 3, 64, [1], "bf16").K[0, :, 0]  # 3 rows of 64
    kr = to_dev(new, "bf16")
    cache.kv_write_rows(0, rows, kr, kr)
    torch.cuda.synchronize()
    case.K[1, 0, 17] = new[0]
    case.V[1, 0, 17] = new[0]
    case.K[0, 1, 3] = new[1]
    case.V[0, 1, 3] = new[1]
    _check_codes(cache, case)
    out, lse = cache.attn_full(0, q, 0.125)
    torch.cuda.synchronize()
    for b, T in enumerate(case.lengths):
        K, V = _dq(case, b, T)
        ref, ref_lse, _ = oracle.full_attention(case.q[b], K, V, 0.125)
        assert_close(host(out[b]), ref, TOL["bf16"], f"out b={b}")


@pytest.mark.parametrize("spec", CASES[1:3], ids=IDS[1:3])
def test_fp8_fused_append_matches_separate_append(spec):
    case, P, sm = _case(spec)
    cache_a = _cache(case, P)
    q, kn, vn = _fill(cache_a, case)
    k_top, rec = 5, 2
    out_f, lse_f = cache_a.attn_full(0, q, sm)
    out_d, lse_d, sel, cnt = cache_a.attn_delta_select(0, q, sm, k_top, rec)
    out_s, lse_s = cache_a.attn_sparse(0, q, sm, sel, cnt)
    k, v = to_dev(case.K, "bf16"), to_dev(case.V, "bf16")
    for tier in ("full", "delta", "sparse"):
        cache_b = _cache(case, P)
        cache_b.seq_reset([n - 1 for n in case.lengths])
        cache_b.kv_prefill(0, k, v)
        cache_b.step_begin()
        if tier == "full":
            o, lse = cache_b.attn_full(0, q, sm, k_new=kn, v_new=vn)
            ref = (out_f, lse_f)
        elif tier == "delta":
            o, lse, s2, c2 = cache_b.attn_delta_select(0, q, sm, k_top, rec, k_new=kn, v_new=vn)
            ref = (out_d, lse_d)
            assert torch.equal(s2, sel) and torch.equal(c2, cnt)
        else:
            o, lse = cache_b.attn_sparse(0, q, sm, sel, cnt, k_new=kn, v_new=vn)
            ref = (out_s, lse_s)
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), tier
        _check_codes(cache_b, case)
