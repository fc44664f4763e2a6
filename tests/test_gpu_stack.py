"""GPU parity of whole decode stacks at the workloads' full sizes, run by bench.py's
own StackBench (the launch configuration the benchmark times).  Sampled batch
rows, layers and steps are recomputed by the oracle from the host recipe."""
import gc

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, LSE_TOL, assert_close, check_selection
from workload import WORKLOADS

pytestmark = pytest.mark.gpu

SAMPLES = {
    # workload: timed/warm-up steps, steps checked, batch rows, layers checked
    "stack28_b8_t16k": dict(warmup=0, steps=256, check=[0, 100, 255], rows=[0, 7], layers=[0, 2, 3, 23, 27]),
    "stack28_b16_t64k": dict(warmup=4, steps=2, check=[4], rows=[0, 15], layers=[0, 2, 3, 23, 27]),
    "stack36_b32_t8k_32k": dict(warmup=4, steps=2, check=[5], rows=None, layers=[0, 2, 3, 34, 35]),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,kv", [("stack28_b8_t16k", None), ("stack28_b16_t64k", None),
                                     ("stack36_b32_t8k_32k", None), ("stack28_b16_t64k", "fp8"),
                                     ("stack36_b32_t8k_32k", "fp8")])
def test_stack_full_size_sampled(name, kv):
    import bench
    from oracle.quant import quantize_dequantize
    wl = WORKLOADS[name]
    spec = SAMPLES[name]
    print(f"stack parity: {wl.name} kv {kv or wl.dtype}", flush=True)
    sb = bench.StackBench(wl, spec["warmup"], spec["steps"], kv_dtype=kv)
    rec, tiers, lens0 = sb.rec, sb.tiers, sb.lens0
    rows = spec["rows"] or [int(np.argmin(lens0)), int(np.argmax(lens0))]
    deltas = [l for l, t in enumerate(tiers) if t == "delta"]
    captured = {}

    def on_step(s, stack):
        if s not in spec["check"]:
            return
        torch.cuda.synchronize()
        cap = {"out": {}, "lse": {}, "sel": {}, "cnt": {}}
        for layer in spec["layers"]:
            cap["out"][layer] = stack.out[layer, rows].float().cpu().numpy().astype(np.float64)
            cap["lse"][layer] = stack.lse[layer, rows].cpu().numpy().astype(np.float64)
        for layer in deltas:
            cap["sel"][layer] = stack.sel[layer][rows].cpu().numpy()
            cap["cnt"][layer] = stack.sel_count[layer][rows].cpu().numpy()
        captured[s] = cap

    sb.run(tiers, on_step=on_step)
    del sb
    gc.collect()
    torch.cuda.empty_cache()
    assert sorted(captured) == spec["check"]

    n_band = 0
    for s, cap in captured.items():
        epoch = rec.epoch_of_step(s)
        for i, b in enumerate(rows):
            T = lens0[b] + s + 1
            for layer in spec["layers"]:
                tier = tiers[layer]
                K, V = rec.layer_kv(layer, b, T, epoch)
                if kv == "fp8":
                    K, V = quantize_dequantize(K), quantize_dequantize(V)
                q = rec.q(layer, s, b)
                got, got_lse = cap["out"][layer][i], cap["lse"][layer][i]
                what = f"{wl.name} step {s} row {b} layer {layer} ({tier})"
                if tier == "full":
                    ref, ref_lse, _ = oracle.full_attention(q, K, V, wl.sm_scale)
                elif tier == "delta":
                    r = oracle.delta_layer(q, K, V, wl.sm_scale, wl.page, wl.k_top, wl.recency)
                    ref, ref_lse = r["out"], r["lse"]
                    for g in range(wl.hkv):
                        n_band += check_selection(cap["sel"][layer][i, g], int(cap["cnt"][layer][i, g]),
                                                  r["page_scores"][g], wl.k_top, wl.recency, wl.k_top + wl.recency)
                else:
                    src = max(d for d in deltas if d < layer)
                    sels = [cap["sel"][src][i, g, :int(cap["cnt"][src][i, g])].tolist() for g in range(wl.hkv)]
                    ref, ref_lse = oracle.sparse_attention(q, K, V, sels, wl.page, wl.sm_scale)
                assert_close(got, ref, TOL[wl.dtype], what)
                assert_close(got_lse, ref_lse, LSE_TOL[wl.dtype], what + " lse")
                del K, V
    print(f"{wl.name}: {n_band} selected pages differ inside the boundary band", flush=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_native_stack_step_equals_python_loop(kv):
    """lak_stack_step (schedule in C++) gives the same bits as the per-layer calls."""
    from layer_aware_kv_amd import DeltaStack, LakError, PagedKVCache
    from workload.cases import random_case
    L, B, HQ, HKV, D, P = 6, 3, 8, 2, 64, 16
    lens = [300, 517, 64]
    tiers = ["full", "full", "delta", "sparse", "delta", "sparse"]
    steps = 5
    runs = []
    for native in (True, False):
        cache = PagedKVCache(L, B, HQ, HKV, D, P, 64, 3 * 64, kv)
        cache.seq_reset(lens, reserve_tokens=steps)
        for layer in range(L):
            c = random_case(100 + layer, B, HQ, HKV, D, lens, "bf16")
            cache.kv_prefill(layer, torch.from_numpy(c.K).to(torch.bfloat16).cuda(),
                             torch.from_numpy(c.V).to(torch.bfloat16).cuda())
        st = DeltaStack(cache, tiers, 3, 2, 0.125, native=native)
        outs = []
        for s in range(steps):
            c = random_case(200 + s, L * B, HQ, HKV, D, [1], "bf16")
            q = torch.from_numpy(c.q).to(torch.bfloat16).cuda().view(L, B, HQ, D)
            kn = torch.from_numpy(c.k_new).to(torch.bfloat16).cuda().view(L, B, HKV, D)
            vn = torch.from_numpy(c.v_new).to(torch.bfloat16).cuda().view(L, B, HKV, D)
            st.step(q, kn, vn)
            outs.append((st.out.clone(), st.lse.clone(), {l: v.clone() for l, v in st.sel.items()}))
        torch.cuda.synchronize()
        runs.append(outs)
    for (o1, l1, s1), (o2, l2, s2) in zip(*runs):
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert all(torch.equal(s1[k], s2[k]) for k in s1)
    # a sparse layer before any delta-layer is refused before anything runs
    cache = PagedKVCache(2, 1, 4, 1, 64, 16, 8, 8, "bf16")
    cache.seq_reset([20], reserve_tokens=4)
    st = DeltaStack.__new__(DeltaStack)
    DeltaStack.__init__(st, cache, ["full", "delta"], 1, 1, 1.0)
    st.tiers = ["full", "sparse"]
    st._desc = None
    z = torch.zeros((2, 1, 4, 64), dtype=torch.bfloat16, device="cuda")
    zk = torch.zeros((2, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(LakError, match="LAK_EINVAL"):
        st.step(z, zk, zk)
    assert cache.seq_lens_host() == [20]  # nothing ran, not even the step's length increment


@pytest.mark.parametrize("native", [True, False])
def test_traced_stack_times_every_decode_kernel(native):
    """Events attached to the decode kernels (timing-only HIP events, as the benchmark
    uses, and torch's default events) leave every output bit unchanged and give each
    kernel a positive duration; one step's kernels fit inside that step's wall time."""
    import time
    from layer_aware_kv_amd import DeltaStack, PagedKVCache
    from layer_aware_kv_amd._lib import TimingEvent, event_elapsed_ms
    from workload.cases import random_case
    L, B, HQ, HKV, D, P = 5, 2, 8, 2, 128, 16
    lens = [700, 333]
    tiers = ["full", "delta", "sparse", "sparse", "full"]

    class Pairs:
        def __init__(self, make):
            self.make, self.records = make, []

        def pair(self, layer, tier):
            ev = (self.make(), self.make())
            self.records.append((layer, tier, ev))
            return ev

    def torch_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()  # torch creates the HIP event at its first record
        return e

    runs = []
    for make in (None, TimingEvent, torch_event):
        cache = PagedKVCache(L, B, HQ, HKV, D, P, 64, 2 * 64, "bf16")
        cache.seq_reset(lens, reserve_tokens=4)
        for layer in range(L):
            c = random_case(300 + layer, B, HQ, HKV, D, lens, "bf16")
            cache.kv_prefill(layer, torch.from_numpy(c.K).to(torch.bfloat16).cuda(),
                             torch.from_numpy(c.V).to(torch.bfloat16).cuda())
        st = DeltaStack(cache, tiers, 4, 2, 0.09, native=native)
        c = random_case(400, L * B, HQ, HKV, D, [1], "bf16")
        q = torch.from_numpy(c.q).to(torch.bfloat16).cuda().view(L, B, HQ, D)
        kn = torch.from_numpy(c.k_new).to(torch.bfloat16).cuda().view(L, B, HKV, D)
        vn = torch.from_numpy(c.v_new).to(torch.bfloat16).cuda().view(L, B, HKV, D)
        tr = Pairs(make) if make is not None else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st.step(q, kn, vn, tr)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        runs.append((st.out.clone(), st.lse.clone(), {l: v.clone() for l, v in st.sel.items()}))
        if tr is not None:
            assert [(l, t) for l, t, _ in tr.records] == list(enumerate(tiers))
            ms = [event_elapsed_ms(*ev) for _, _, ev in tr.records]
            print(make.__name__, [round(x * 1e3, 1) for x in ms], f"wall {wall_ms:.3f} ms", flush=True)
            assert all(0.0 < x < wall_ms for x in ms)
            assert sum(ms) < wall_ms
    for o, l, s in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])
        assert all(torch.equal(s[k], runs[0][2][k]) for k in s)
