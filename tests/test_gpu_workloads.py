"""GPU tests on the five decode workloads: the device generator reproduces the host
recipe exactly, and the workloads' layers match the oracle (full sizes sampled)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, LSE_TOL, assert_close, check_selection, host
from workload import recipe_for, WORKLOADS
from workload import philox as px

pytestmark = pytest.mark.gpu


def _dev(name, strength=None):
    import dataclasses
    from workload import Recipe
    from workload.device import DeviceInputs
    if strength is None:
        return DeviceInputs(recipe_for(name))
    return DeviceInputs(Recipe(dataclasses.replace(WORKLOADS[name], salient_strength=strength)))


@pytest.mark.parametrize("name,strength", [("layer1_f32_b1_t1k", None), ("layer1_bf16_b1_t8k", None),
                                           ("stack36_b32_t8k_32k", None), ("layer1_bf16_b1_t8k", 6.3)])
def test_device_generator_equals_host(name, strength):
    d = _dev(name, strength)
    r, wl = d.r, d.wl
    T = min(wl.context, 3000)
    k = torch.empty((wl.batch, wl.hkv, T, wl.d), dtype=d.torch_dtype, device="cuda")
    v = torch.empty_like(k)
    sal_epoch0 = d.salient_positions(0)
    d.fill_kv(0, k, v, T)
    q = torch.empty((3, wl.batch, wl.hq, wl.d), dtype=d.torch_dtype, device="cuda")
    d.fill_queries(0, 5, 3, q)
    kn = torch.empty((2, wl.batch, wl.hkv, wl.d), dtype=d.torch_dtype, device="cuda")
    vn = torch.empty_like(kn)
    d.fill_new_kv(0, 7, 2, kn, vn)
    torch.cuda.synchronize()
    for b in sorted({0, wl.batch - 1}):
        for g in sorted({0, wl.hkv - 1}):
            # positions beyond T are outside this fill; salient positions < T are applied
            exp_k = r.k_rows(0, b, g, 0, T)
            assert np.array_equal(host(k[b, g]), exp_k)
            assert np.array_equal(host(v[b, g]), r.v_rows(0, b, g, 0, T))
            t_new = int(r.lengths0()[b]) + 7
            assert np.array_equal(host(kn[0, b, g]), r.k_rows(0, b, g, t_new, t_new + 1)[0])
        for s in range(3):
            assert np.array_equal(host(q[s, b]), r.q(0, 5 + s, b))


def _run_single_layer(name):
    """The single-layer workloads: one layer run as full, delta-select and sparse."""
    from layer_aware_kv_amd import PagedKVCache
    d = _dev(name)
    r, wl = d.r, d.wl
    T = wl.context
    cache = PagedKVCache(1, wl.batch, wl.hq, wl.hkv, wl.d, wl.page, wl.max_pages_per_seq() + 1,
                         wl.batch * (wl.max_pages_per_seq() + 1), wl.dtype)
    cache.seq_reset([T - 1] * wl.batch, reserve_tokens=1)
    k = torch.empty((wl.batch, wl.hkv, T, wl.d), dtype=d.torch_dtype, device="cuda")
    v = torch.empty_like(k)
    d.fill_kv(0, k, v, T)
    cache.kv_prefill(0, k, v)
    cache.step_begin()
    cache.kv_append(0, k[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous())
    q = torch.empty((1, wl.batch, wl.hq, wl.d), dtype=d.torch_dtype, device="cuda")
    d.fill_queries(0, 0, 1, q)
    return d, cache, q[0]


@pytest.mark.parametrize("name", ["layer1_f32_b1_t1k", "layer1_bf16_b1_t8k"])
def test_single_layer_workload_full_delta_sparse(name):
    d, cache, q = _run_single_layer(name)
    r, wl = d.r, d.wl
    T = wl.context
    salient = wl.q_mode == "salient"
    aggs = ["max"] if salient else ["max", "sum"]
    for agg in aggs:
        scores = torch.zeros((wl.batch, wl.hkv, cache.max_pages), device="cuda")
        out_f, lse_f = cache.attn_full(0, q, wl.sm_scale)
        out_d, lse_d, sel, cnt = cache.attn_delta_select(0, q, wl.sm_scale, wl.k_top, wl.recency, agg,
                                                         page_scores=scores)
        out_s, lse_s = cache.attn_sparse(0, q, wl.sm_scale, sel, cnt)
        torch.cuda.synchronize()
        K, V = r.layer_kv(0, 0, T)
        qh = r.q(0, 0, 0)
        ref = oracle.delta_layer(qh, K, V, wl.sm_scale, wl.page, wl.k_top, wl.recency, agg)
        assert_close(host(out_f[0]), ref["out"], TOL[wl.dtype], "full")
        assert_close(host(lse_f[0]), ref["lse"], LSE_TOL[wl.dtype], "lse")
        assert torch.equal(out_d, out_f)
        NP = -(-T // wl.page)
        # MAX: fp16 weights relative to each (head, sub-tile) maximum, relative error <= 2^-11
        np.testing.assert_allclose(scores[0, :, :NP].cpu().numpy(), ref["page_scores"],
                                   rtol=6e-4 if agg == "max" else 1e-4, atol=1e-7)
        for g in range(wl.hkv):
            check_selection(sel[0, g].cpu().numpy(), int(cnt[0, g]), ref["page_scores"][g], wl.k_top, wl.recency,
                            sel.shape[-1])
        sels = [sel[0, g, :int(cnt[0, g])].cpu().tolist() for g in range(wl.hkv)]
        ref_s, ref_ls = oracle.sparse_attention(qh, K, V, sels, wl.page, wl.sm_scale)
        assert_close(host(out_s[0]), ref_s, TOL[wl.dtype], "sparse")
        assert_close(host(lse_s[0]), ref_ls, LSE_TOL[wl.dtype], "sparse lse")
        if salient:
            # the salient far keys are in the selection of every group
            for g in range(wl.hkv):
                sal_pages = {p // wl.page for p in r.salient_slots(0, g, 0)}
                assert len(sal_pages & set(sels[g])) >= len(sal_pages) * 3 // 4
