"""Seeded random sweep of small configurations through the C ABI against the oracle:
batch, ragged lengths (including 0-page-boundary cases), group size, head dim, page
size, pool element type, budget, aggregation and scope are drawn per case, then one
decode step runs full, delta-select and sparse attention on the same cache."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant as Q
from tests.gpu_util import LSE_TOL, TOL, assert_close, check_selection, host, to_dev
from workload.cases import plant_salient, random_case

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(i):
    rng = np.random.default_rng(7000 + i)
    kv = ["bf16", "f32", "fp8"][i % 3]
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    hkv = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(1, 1500, size=B)]
    if rng.random() < 0.5:  # a length on a page boundary and one just past it
        lens[0] = P * int(rng.integers(1, 20))
        if B > 1:
            lens[1] = P * int(rng.integers(1, 20)) + 1
    NPmax = -(-max(lens) // P)
    k_top = int(rng.integers(0, NPmax + 3))
    rec = int(rng.integers(0, 6))
    if k_top + rec == 0:
        rec = 1
    agg = str(rng.choice(["max", "sum"]))
    scope = str(rng.choice(["group", "all"]))
    return dict(kv=kv, D=D, G=G, hkv=hkv, P=P, B=B, lens=lens, k_top=k_top, rec=rec, agg=agg, scope=scope,
                seed=int(rng.integers(1, 10 ** 6)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    from layer_aware_kv_amd import PagedKVCache
    c = _draw(i)
    print(c, flush=True)
    kv, D, G, hkv, P, B, lens = c["kv"], c["D"], c["G"], c["hkv"], c["P"], c["B"], c["lens"]
    hq = G * hkv
    act = "bf16" if kv == "fp8" else kv
    case = random_case(c["seed"], B, hq, hkv, D, lens, act)
    for b in range(B):
        if lens[b] > 64:
            plant_salient(case, b, 0, [lens[b] // 5, lens[b] // 2], G)
    sm = float(1.0 / np.sqrt(D))
    max_pages = max(-(-n // P) for n in lens) + 1
    cache = PagedKVCache(1, B, hq, hkv, D, P, max_pages, sum(-(-n // P) for n in lens) + 2, kv)
    cache.seq_reset([n - 1 for n in lens])
    k, v = to_dev(case.K, act), to_dev(case.V, act)
    cache.kv_prefill(0, k, v)
    cache.step_begin()
    kn = torch.stack([k[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    vn = torch.stack([v[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    q = to_dev(case.q, act)
    k_top, rec, agg, scope = c["k_top"], c["rec"], c["agg"], c["scope"]
    R = cache.sel_rows(scope)
    # the delta call appends this step's token (fused), the others read it from the pool
    out_d, lse_d, sel, cnt = cache.attn_delta_select(0, q, sm, k_top, rec, agg, scope, k_new=kn, v_new=vn)
    out_f, lse_f = cache.attn_full(0, q, sm)
    out_s, lse_s = cache.attn_sparse(0, q, sm, sel, cnt, scope)
    torch.cuda.synchronize()
    assert torch.equal(out_d, out_f) and torch.equal(lse_d, lse_f)
    tol = TOL["f32" if kv == "f32" else "bf16"]
    ltol = LSE_TOL["f32" if kv == "f32" else "bf16"]
    for b, T in enumerate(lens):
        K, V = case.K[b, :, :T], case.V[b, :, :T]
        if kv == "fp8":
            K, V = Q.quantize_dequantize(K), Q.quantize_dequantize(V)
        r = oracle.delta_layer(case.q[b], K, V, sm, P, k_top, rec, agg, scope)
        assert_close(host(out_f[b]), r["out"], tol, f"full b={b}")
        assert_close(host(lse_f[b]), r["lse"], ltol, f"lse b={b}")
        for row in range(R):
            check_selection(sel[b, row].cpu().numpy(), int(cnt[b, row]), r["page_scores"][row], k_top, rec,
                            sel.shape[-1])
        sels = [sel[b, g if R > 1 else 0, :int(cnt[b, g if R > 1 else 0])].cpu().tolist() for g in range(hkv)]
        ref, ref_lse = oracle.sparse_attention(case.q[b], K, V, sels, P, sm)
        assert_close(host(out_s[b]), ref, tol, f"sparse b={b}")
        assert_close(host(lse_s[b]), ref_lse, ltol, f"sparse lse b={b}")
