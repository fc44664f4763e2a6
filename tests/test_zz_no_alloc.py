"""lak_attn_sparse_noalloc (split partials in the library's static device scratch, for
callers that cannot allocate) against lak_attn_sparse, which takes the caller's
workspace: the same kernels and split plan, so the same bits.  Two calls in a row on
the same GPU, the second on a smaller input, then a call too large for the scratch."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, LSE_TOL, assert_close, fill_and_step, host, make_cache, to_dev
from workload.cases import random_case, plant_salient

pytestmark = pytest.mark.gpu

# (dtype, B, Hq, Hkv, D, P, lengths, k_top, recency): the larger input first
CALLS = [("bf16", 6, 28, 4, 128, 16, [1, 15, 16, 17, 1000, 4097], 60, 4),
         ("bf16", 2, 8, 2, 64, 32, [100, 700], 5, 2)]


def _one(spec, seed):
    dtype, B, HQ, HKV, D, P, lens, k_top, rec = spec
    print(f"noalloc case B={B} Hq={HQ} Hkv={HKV} D={D} P={P} lens={lens}", flush=True)
    case = random_case(seed, B, HQ, HKV, D, lens, dtype)
    for b, T in enumerate(lens):
        if T > 64:
            plant_salient(case, b, 0, [T // 5, T // 2], HQ // HKV)
    cache = make_cache(case, P)
    q = fill_and_step(cache, case)
    sm = float(1.0 / np.sqrt(D))
    _, _, sel, cnt = cache.attn_delta_select(0, q, sm, k_top, rec)
    out_ws, lse_ws = cache.attn_sparse(0, q, sm, sel, cnt)
    out_na = torch.full_like(out_ws, 7.0)
    lse_na = torch.full_like(lse_ws, 7.0)
    cache.attn_sparse_noalloc(0, q, sm, sel, cnt, out=out_na, lse=lse_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws)
    for b, T in enumerate(lens):
        sels = [sel[b, g, :int(cnt[b, g])].cpu().tolist() for g in range(HKV)]
        ref, ref_lse = oracle.sparse_attention(case.q[b], case.K[b, :, :T], case.V[b, :, :T], sels, P, sm)
        assert_close(host(out_na[b]), ref, TOL[dtype], f"noalloc out b={b}")
        assert_close(host(lse_na[b]), ref_lse, LSE_TOL[dtype], f"noalloc lse b={b}")


def test_noalloc_sparse_equals_workspace_call_twice():
    for i, spec in enumerate(CALLS):
        _one(spec, 40 + i)


def test_noalloc_sparse_rejects_calls_beyond_its_scratch():
    """One row of 4096 pages among 15 short ones: the planner gives that row ~200 splits,
    so the partials (16 x 16 heads x ~200 splits x 128 x 4 bytes) exceed 16 MiB."""
    from layer_aware_kv_amd import LakError, PagedKVCache
    B, HQ, HKV, D, P = 16, 16, 1, 128, 16
    lens = [4096 * P] + [P] * (B - 1)
    cache = PagedKVCache(1, B, HQ, HKV, D, P, 4097, 4096 + B, "bf16")
    cache.seq_reset(lens)
    q = torch.zeros((B, HQ, D), dtype=torch.bfloat16, device="cuda")
    sel = torch.arange(4096, dtype=torch.int32, device="cuda").repeat(B, HKV, 1).contiguous()
    cnt = torch.tensor([[4096]] + [[1]] * (B - 1), dtype=torch.int32, device="cuda")
    out = torch.full((B, HQ, D), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, HQ), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(LakError, match="LAK_EINVAL.*static scratch"):
        cache.attn_sparse_noalloc(0, q, 0.1, sel, cnt, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out == 3.0).all() and (lse == 3.0).all()  # nothing was enqueued


@pytest.mark.parametrize("kv", ["fp8", "f32"])
def test_noalloc_sparse_other_pool_types(kv):
    """The same comparison on fp8 (E4M3 codes + row scales) and float32 pools."""
    from layer_aware_kv_amd import PagedKVCache
    from oracle import quant as Q
    act = "bf16" if kv == "fp8" else kv
    B, HQ, HKV, D, P = 3, 16, 2, 128, 16
    lens = [700, 33, 1500]
    print(f"noalloc case kv={kv} lens={lens}", flush=True)
    case = random_case(77, B, HQ, HKV, D, lens, act)
    cache = PagedKVCache(1, B, HQ, HKV, D, P, 100, 3 * 100, kv)
    cache.seq_reset([n - 1 for n in lens])
    k, v = to_dev(case.K, act), to_dev(case.V, act)
    cache.kv_prefill(0, k, v)
    cache.step_begin()
    kn = torch.stack([k[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    vn = torch.stack([v[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    cache.kv_append(0, kn, vn)
    q = to_dev(case.q, act)
    sm = float(1.0 / np.sqrt(D))
    _, _, sel, cnt = cache.attn_delta_select(0, q, sm, 20, 3)
    out_ws, lse_ws = cache.attn_sparse(0, q, sm, sel, cnt)
    out_na, lse_na = cache.attn_sparse_noalloc(0, q, sm, sel, cnt)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws)
    for b, T in enumerate(lens):
        K, V = case.K[b, :, :T], case.V[b, :, :T]
        if kv == "fp8":
            K, V = Q.quantize_dequantize(K), Q.quantize_dequantize(V)
        sels = [sel[b, g, :int(cnt[b, g])].cpu().tolist() for g in range(HKV)]
        ref, _ = oracle.sparse_attention(case.q[b], K, V, sels, P, sm)
        assert_close(host(out_na[b]), ref, TOL["f32" if kv == "f32" else "bf16"], f"noalloc {kv} b={b}")
