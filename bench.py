#!/usr/bin/env python3
"""Decode-attention throughput of DELTA's three-tier layer stack on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload stack28_b16_t64k] [--no-cpu-baseline]

Workload (default): the 28-layer attention-only decode stack at long reasoning
length -- batch 16, context 65536 tokens, 28 query / 4 KV heads, head dim 128,
page 16, bf16; layers 0-1 full, delta-layers 2, 9, 16, 23, the other 22 layers
sparse over a 4096-token budget (192 top-k pages + 64 recency pages).  All inputs
(prefilled KV cache, every step's queries and appended keys/values) are generated
on the device before timing, so they are resident in HBM.

A step = one decode step of the whole stack: page-table step, KV append, and
full / delta-select / sparse attention in every layer.  Timed: exactly K steps
after W warm-up steps, bracketed by torch.cuda.synchronize().

Printed: one JSON line.  value = B * K / elapsed (decode tokens/s of the DELTA
stack).  Also the all-full-attention stack on the same inputs, per-tier decode
kernel durations (HIP events recorded by the library around its decode kernel),
the HBM roofline of the dominant kernel, and the CPU oracle's throughput on a
bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention tokens/s per stack + achieved HBM GB/s (full vs sparse layers)"
PEAK_HBM_GBPS = 8000.0
KERNEL_NAMES = {
    "full": "lak::decode_kernel<{esz}, 128, MODE_FULL>",
    "delta": "lak::decode_kernel<{esz}, 128, MODE_DELTA>",
    "sparse": "lak::decode_kernel<{esz}, 128, MODE_SPARSE>",
}
KV_ESZ = {"bf16": 2, "f32": 4, "fp8": 1}
STACK_WORKLOADS = ["stack28_b8_t16k", "stack28_b16_t64k", "stack36_b32_t8k_32k"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in ("layer_aware_kv_amd/csrc/decode_kernels.hip", "layer_aware_kv_amd/csrc/lak_device.h",
                "layer_aware_kv_amd/csrc/lak_internal.h", "layer_aware_kv_amd/csrc/api.hip",
                "layer_aware_kv_amd/build.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Tracer:
    """Hands out pre-created event pairs for the decode kernels of chosen tiers.  The
    events are timing-only HIP events (no system-scope fence when recorded: with torch's
    default events each attached pair cost the stream ~5 us, 0.7% of a workload-3 step
    with events on its 4 delta decodes and 2.8% of a workload-4 step with events on its
    29 sparse decodes; these cost 0.2% and 1%)."""

    def __init__(self, torch, tiers, n_pairs):
        from layer_aware_kv_amd._lib import TimingEvent
        self.tiers = set(tiers)
        self.pool = [(TimingEvent(), TimingEvent()) for _ in range(n_pairs)]
        self.used = 0
        self.step = 0
        self.records = []  # (step, layer, tier, (ev0, ev1))

    def pair(self, layer, tier):
        if tier not in self.tiers or self.used >= len(self.pool):
            return None
        ev = self.pool[self.used]
        self.used += 1
        self.records.append((self.step, layer, tier, ev))
        return ev


class StackBench:
    """Device set-up and the step loop of one stack workload (inputs resident in HBM)."""

    def __init__(self, wl, warmup, steps, agg="max", scope="group", kv_dtype=None):
        import torch
        from layer_aware_kv_amd import PagedKVCache, layer_tiers
        from workload import Recipe
        from workload.device import DeviceInputs

        self.torch = torch
        self.wl = wl
        self.agg, self.scope = agg, scope
        self.W, self.K = warmup, steps
        self.S = warmup + steps
        self.rec = Recipe(wl)
        self.dev = DeviceInputs(self.rec)
        self.lens0 = [int(x) for x in self.rec.lengths0()]
        self.tiers = layer_tiers(wl.num_layers, wl.full_layers, wl.delta_layers)
        B, L, P = wl.batch, wl.num_layers, wl.page
        max_pages = math.ceil((max(self.lens0) + self.S) / P) + 1
        num_pages = sum(math.ceil((t + self.S) / P) for t in self.lens0)
        self.kv_dtype = kv_dtype or wl.dtype
        self.cache = PagedKVCache(L, B, wl.hq, wl.hkv, wl.d, P, max_pages, num_pages, self.kv_dtype)
        self.cache.seq_reset(self.lens0, reserve_tokens=self.S)
        self.dirty = False
        self.prefill_all()
        td = self.dev.torch_dtype
        S = self.S
        self.Q = torch.empty((S, L, B, wl.hq, wl.d), dtype=td, device="cuda")
        self.KN = torch.empty((S, L, B, wl.hkv, wl.d), dtype=td, device="cuda")
        self.VN = torch.empty_like(self.KN)
        tq = torch.empty((S, B, wl.hq, wl.d), dtype=td, device="cuda")
        tk = torch.empty((S, B, wl.hkv, wl.d), dtype=td, device="cuda")
        tv = torch.empty_like(tk)
        for layer in range(L):
            self.dev.fill_queries(layer, 0, S, tq)
            self.Q[:, layer] = tq
            self.dev.fill_new_kv(layer, 0, S, tk, tv)
            self.KN[:, layer] = tk
            self.VN[:, layer] = tv
        self.drift = {}
        if wl.drift_every:
            for s in range(wl.drift_every, S, wl.drift_every):
                self.drift[s] = [self.dev.drift_rows(layer, s // wl.drift_every) for layer in range(L)]
        torch.cuda.synchronize()

    def prefill_all(self):
        torch, wl = self.torch, self.wl
        tmax = max(self.lens0)
        kst = torch.empty((wl.batch, wl.hkv, tmax, wl.d), dtype=self.dev.torch_dtype, device="cuda")
        vst = torch.empty_like(kst)
        for layer in range(wl.num_layers):
            self.dev.fill_kv(layer, kst, vst, tmax, epoch=0)
            self.cache.kv_prefill(layer, kst, vst)
        torch.cuda.synchronize()
        self.dirty = False

    def run(self, tiers, tracer=None, on_step=None):
        """W untimed steps, then K timed steps; returns the timed seconds.  ``on_step(s,
        stack)`` (tests only) runs after every step and is not meant for timing."""
        from layer_aware_kv_amd import DeltaStack
        torch, wl, cache = self.torch, self.wl, self.cache
        cache.seq_reset(self.lens0, reserve_tokens=self.S)
        if self.dirty:  # a drift event rewrote keys: restore the prefilled state
            self.prefill_all()
        stack = DeltaStack(cache, tiers, wl.k_top, wl.recency, wl.sm_scale, self.agg, self.scope)

        def one(s, tr):
            if s in self.drift:
                for layer, (rows, krows) in enumerate(self.drift[s]):
                    if rows is not None:
                        cache.kv_write_rows(layer, rows, krows)
                self.dirty = True
            if tr is not None:
                tr.step = s
            stack.step(self.Q[s], self.KN[s], self.VN[s], tr)
            if on_step is not None:
                on_step(s, stack)

        for s in range(self.W):
            one(s, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(self.W, self.S):
            one(s, tracer)
        torch.cuda.synchronize()
        return time.perf_counter() - t0


def traffic_for(wl, dom, kv_dtype):
    """Counter-measured HBM bytes per launch of the dominant kernel, from the committed
    counter summary, while the kernel sources still hash to the value it was taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    try:
        with open(TRAFFIC_FILE) as f:
            tj = json.load(f)
        ent = tj.get("kernels", {}).get(dom)
        if (tj.get("source_hash") == kernel_source_hash() and tj.get("workload") == wl.name and ent
                and tj.get("kv_dtype", wl.dtype) == kv_dtype):
            return ent["hbm_bytes_per_launch"], (f"profiles/traffic.json: rocprofv3 FETCH_SIZE / WRITE_SIZE "
                                                 f"counters taken on kernel sources {tj['source_hash']} "
                                                 f"(the current ones), not in this run")
    except (OSError, ValueError, KeyError):
        pass
    return None, None


def measure_stack(torch, wl, W, K, agg="max", scope="group", kv_dtype=None, keep=False):
    """Times one stack workload: the DELTA stack (value), a per-tier pass with events on
    every decode kernel, and the same stack with every layer full.  Returns the summary
    and, with ``keep``, the StackBench (for the fidelity pass)."""
    from layer_aware_kv_amd import accounting as acc
    from layer_aware_kv_amd._lib import event_elapsed_ms

    B, L, HQ, HKV, D, P = wl.batch, wl.num_layers, wl.hq, wl.hkv, wl.d, wl.page
    e = 2 if wl.dtype == "bf16" else 4
    kv_dtype = kv_dtype or wl.dtype
    kv_row = acc.kv_row_bytes(D, kv_dtype)
    t_setup = time.perf_counter()
    sb = StackBench(wl, W, K, agg=agg, scope=scope, kv_dtype=kv_dtype)
    lens0, tiers = sb.lens0, sb.tiers
    pool_gb = 2 * L * sb.cache.k_pools[0].numel() * sb.cache.k_pools[0].element_size() / 1e9
    log(f"{wl.name}: set-up {time.perf_counter() - t_setup:.1f} s, {pool_gb:.1f} GB of {kv_dtype} KV pools, "
        f"W={W} K={K}, drift events at steps {sorted(sb.drift)}")

    # decode-kernel bytes of one launch at step s
    def kernel_bytes(tier, s):
        lens = [t + s + 1 for t in lens0]
        q_bytes = B * HQ * D * e
        if tier == "sparse":
            toks = sum(acc.selected_tokens(t, P, wl.k_top, wl.recency) for t in lens)
            return toks * HKV * kv_row * 2 + q_bytes + B * HKV * (wl.k_top + wl.recency) * 4
        return sum(lens) * HKV * kv_row * 2 + q_bytes

    mid = [t + W + K // 2 + 1 for t in lens0]
    step_bytes = acc.stack_bytes(mid, tiers, HQ, HKV, D, e, P, wl.k_top, wl.recency, kv_row)
    present = sorted(set(tiers))
    dom = max(present, key=lambda t: step_bytes[t])

    # A: the timed DELTA stack, events on the dominant tier's decode kernels
    trA = Tracer(torch, [dom], K * tiers.count(dom))
    tA = sb.run(tiers, trA)
    value = B * K / tA
    log(f"{wl.name}: DELTA stack {tA / K * 1e3:.3f} ms/step, {value:.0f} tok/s")

    def summarize(records):
        out = {}
        for s, layer, tier, (e0, e1) in records:
            d = out.setdefault(tier, {"launches": 0, "ms": 0.0, "bytes": 0})
            d["launches"] += 1
            d["ms"] += event_elapsed_ms(e0, e1)
            d["bytes"] += kernel_bytes(tier, s)
        for tier, d in out.items():
            d["us_per_launch"] = 1e3 * d["ms"] / d["launches"]
            d["achieved_GBps"] = d["bytes"] / (d["ms"] * 1e-3) / 1e9
            d["bytes_per_launch"] = d["bytes"] / d["launches"]
            d["frac_of_peak"] = d["achieved_GBps"] / PEAK_HBM_GBPS
        return out

    domA = summarize(trA.records)[dom]

    # B: per-tier breakdown (events on every decode kernel)
    trB = Tracer(torch, present, K * L)
    sb.run(tiers, trB)
    per_tier = summarize(trB.records)
    for t, d in per_tier.items():
        d["ms_per_step"] = d["ms"] / K
    log(f"{wl.name}: tiers " + ", ".join(f"{t} {d['us_per_launch']:.1f} us {d['achieved_GBps']:.0f} GB/s"
                                         for t, d in sorted(per_tier.items())))

    # C: the same stack with every layer full, same inputs
    tC = sb.run(["full"] * L)
    full_value = B * K / tC
    log(f"{wl.name}: all-full stack {tC / K * 1e3:.3f} ms/step, {full_value:.0f} tok/s")

    attended_delta = acc.attended_tokens(mid, tiers, P, wl.k_top, wl.recency)
    attended_full = acc.attended_tokens(mid, ["full"] * L, P, wl.k_top, wl.recency)
    traffic, traffic_src = traffic_for(wl, dom, kv_dtype)
    summary = {
        "tokens_per_s": value,
        "ms_per_step": tA / K * 1e3,
        "steps": K,
        "warmup": W,
        "roofline": {
            "bound": "hbm",
            "kernel": KERNEL_NAMES[dom].format(esz=KV_ESZ[kv_dtype]),
            "achieved": round(domA["achieved_GBps"], 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(domA["achieved_GBps"] / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "bytes_per_launch": int(domA["bytes_per_launch"]),
            "us_per_launch": round(domA["us_per_launch"], 2),
            "launches": domA["launches"],
            "timing": "HIP events attached to each launch of the kernel (its start and end)",
        },
        "tiers": {t: {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}
                  for t, d in per_tier.items()},
        "all_full_tokens_per_s": round(full_value, 2),
        "all_full_ms_per_step": round(tC / K * 1e3, 4),
        "speedup_vs_all_full": round(value / full_value, 4),
        "attended_token_ratio": round(attended_full / attended_delta, 4),
        "algorithmic_bytes_per_step": {t: int(v) for t, v in step_bytes.items()},
        "stack_GBps": round(sum(step_bytes.values()) / (tA / K) / 1e9, 1),
    }
    if keep:
        return summary, sb
    del sb
    torch.cuda.empty_cache()
    return summary, None


def workload_config(wl, args_agg="max", args_scope="group", kv_dtype=None):
    return {
        "workload": wl.name,
        "layers": wl.num_layers, "batch": wl.batch, "context": wl.context, "q_heads": wl.hq,
        "kv_heads": wl.hkv, "head_dim": wl.d, "page": wl.page, "top_k_pages": wl.k_top,
        "recency_pages": wl.recency, "full_layers": list(wl.full_layers), "delta_layers": list(wl.delta_layers),
        "ragged_min": wl.ragged_min, "agg": args_agg, "scope": args_scope, "kv_dtype": kv_dtype or wl.dtype,
        "salient_strength": wl.salient_strength, "drift_every": wl.drift_every,
        "parallelism": "single GPU",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="stack28_b16_t64k", choices=STACK_WORKLOADS,
                    help="layer-stack workload (default: batch 16 at context 65536)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other stack workloads (timed after the headline one at their own steps)")
    ap.add_argument("--no-fidelity", action="store_true", help="skip the selection-fidelity passes")
    ap.add_argument("--cpu-rows", type=int, default=4, help="batch rows in the CPU oracle sample")
    ap.add_argument("--agg", choices=["max", "sum"], default="max",
                    help="head aggregation of the delta-layers (max: the pages' rule)")
    ap.add_argument("--scope", choices=["group", "all"], default="group",
                    help="heads aggregated per selection: each KV group, or all query heads")
    ap.add_argument("--delta-layers", default=None,
                    help="comma-separated delta-layer list replacing the workload's (sweeps)")
    ap.add_argument("--salient-strength", type=float, default=None,
                    help="salient keys = strength * direction + noise (workload default 4; the fidelity study's "
                         "attention sharpness)")
    ap.add_argument("--sharp-strength", type=float, default=10.0,
                    help="the second, sharper salient strength of the fidelity block")
    ap.add_argument("--kv-dtype", choices=["bf16", "fp8"], default=None,
                    help="KV pool element type (default: the workload's; fp8 = E4M3 codes + per-row scales)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (for HBM counter scaling)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "dispatches": 3}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world > 1:
        print("bench.py runs on one GPU only (--gpus must be 1): sequences and, with per-group "
              "selection, KV heads are independent, so the path would shard by batch or KV head with no "
              "exchange; it is measured here on one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch
    from workload import get

    wl = get(args.workload)
    custom = args.delta_layers is not None or args.salient_strength is not None
    if args.delta_layers is not None:
        wl = dataclasses.replace(wl, delta_layers=tuple(int(x) for x in args.delta_layers.split(",") if x != ""))
    if args.salient_strength is not None:
        wl = dataclasses.replace(wl, salient_strength=args.salient_strength)
    W = wl.warmup if args.warmup is None else args.warmup
    K = wl.steps if args.steps is None else args.steps
    kv_dtype = args.kv_dtype or wl.dtype
    if kv_dtype == "fp8" and wl.dtype != "bf16":
        sys.exit("fp8 pools take bfloat16 rows: use a bf16 workload")
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({props.multi_processor_count} CUs), workload {wl.name}, W={W} K={K}")

    head, sb = measure_stack(torch, wl, W, K, args.agg, args.scope, kv_dtype, keep=not args.no_fidelity)
    result = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded Philox inputs generated on the device; no datasets or weights)",
        "config": workload_config(wl, args.agg, args.scope, kv_dtype),
    }
    result.update({k: v for k, v in head.items() if k not in ("tokens_per_s", "ms_per_step", "steps", "warmup")})
    result["device"] = props.name

    # D: selection fidelity (untimed): at sampled steps every sparse layer is also run
    # with full attention on the same query; recall = exp(lse_sparse - lse_full).  Once on
    # the timed inputs, once with sharper attention (stronger salient keys).
    if not args.no_fidelity:
        fid = [dict(salient_strength=wl.salient_strength, **fidelity_pass(sb, torch))]
        del sb
        torch.cuda.empty_cache()
        if args.sharp_strength and args.sharp_strength != wl.salient_strength:
            wl_s = dataclasses.replace(wl, salient_strength=args.sharp_strength)
            sb_s = StackBench(wl_s, W, K, agg=args.agg, scope=args.scope, kv_dtype=kv_dtype)
            fid.append(dict(salient_strength=args.sharp_strength, **fidelity_pass(sb_s, torch)))
            del sb_s
            torch.cuda.empty_cache()
        for f in fid:
            if "recall_mean" not in f:
                continue
            log("fidelity at salient strength {salient_strength}: recall mean {recall_mean}, p05 {recall_p05}, "
                "min {recall_min}; max |out err| {max_abs_out_err}".format(**f))
        result["fidelity"] = fid

    # E: the other stack workloads, each at its own step count (timed too)
    if not args.no_workloads and not custom:
        result["workloads"] = {}
        for name in STACK_WORKLOADS:
            if name == wl.name:
                continue
            w2 = get(name)
            summ, _ = measure_stack(torch, w2, w2.warmup, w2.steps, args.agg, args.scope, None)
            summ["config"] = workload_config(w2, args.agg, args.scope)
            summ["tokens_per_s"] = round(summ["tokens_per_s"], 2)
            summ["ms_per_step"] = round(summ["ms_per_step"], 4)
            result["workloads"][name] = summ

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, Recipe_of(wl), sb_tiers(wl), W, args.cpu_rows, kv_dtype)
    print(json.dumps(result), flush=True)


def Recipe_of(wl):
    from workload import Recipe
    return Recipe(wl)


def sb_tiers(wl):
    from layer_aware_kv_amd import layer_tiers
    return layer_tiers(wl.num_layers, wl.full_layers, wl.delta_layers)


def fidelity_pass(sb, torch):
    """Attention-mass recall of the selections and sparse-vs-full output error, per
    sparse layer, at the first and last timed steps and around drift events."""
    from layer_aware_kv_amd import fidelity
    wl, cache = sb.wl, sb.cache
    sample = {sb.W, sb.S - 1}
    for s in sb.drift:
        sample |= {s - 1, s}
    sample = {s for s in sample if 0 <= s < sb.S}
    sparse = [l for l, t in enumerate(sb.tiers) if t == "sparse"]
    recalls, errors = {}, {}

    def on_step(s, stack):
        if s not in sample:
            return
        B = cache.batch
        for layer in sparse:
            out_f, lse_f = cache.attn_full(layer, sb.Q[s][layer], wl.sm_scale)
            recalls[(s, layer)] = fidelity.selection_recall(stack.lse[layer, :B], lse_f)
            errors[(s, layer)] = (stack.out[layer, :B].float() - out_f.float()).abs().amax(dim=-1)

    sb.run(sb.tiers, on_step=on_step)
    torch.cuda.synchronize()
    return fidelity.summarize(recalls, errors)


def cpu_baseline(wl, rec, tiers, step, rows, kv_dtype, repeats=3):
    """The CPU oracle, as it stands, on a bounded sample: one whole decode step (every
    layer of the stack, in order) for batch rows 0 .. rows-1, each step run ``repeats``
    times (median per row).  Each tier's layers run on
    the inputs of that tier's first layer (the oracle's work does not depend on the
    values, and generating every layer's keys and values on the host would take longer
    than the timing); sparse layers use the selection of the preceding delta layer.
    fp8 pools: the rows are encoded and decoded by the oracle before timing (the cache
    holds them encoded), and attention runs on the decoded values."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    cores = len(os.sched_getaffinity(0))
    first = {t: tiers.index(t) for t in ("full", "delta", "sparse") if t in tiers}
    times = {t: [] for t in first}
    epoch = rec.epoch_of_step(step)
    total = 0.0      # all oracle time
    per_row = []     # median seconds of one row's step
    log(f"cpu baseline: {rows} row(s) x {len(tiers)} layers x {repeats} runs, {cores} cores")
    with threadpool_limits(limits=cores):
        for b in range(rows):
            T = int(rec.lengths0()[b]) + step + 1
            data = {}
            for t, layer in first.items():
                K, V = rec.layer_kv(layer, b, T, epoch)
                if kv_dtype == "fp8":
                    K, V = oracle.quant.quantize_dequantize(K), oracle.quant.quantize_dequantize(V)
                data[t] = (rec.q(layer, step, b), K, V)
            runs = []
            for _ in range(repeats):
                sel = None
                t_step = 0.0
                for t in tiers:
                    q, K, V = data[t]
                    t0 = time.perf_counter()
                    if t == "full":
                        oracle.full_attention(q, K, V, wl.sm_scale)
                    elif t == "delta":
                        sel = oracle.delta_layer(q, K, V, wl.sm_scale, wl.page, wl.k_top, wl.recency)["sel"]
                    else:
                        oracle.sparse_attention(q, K, V, sel, wl.page, wl.sm_scale)
                    dt = time.perf_counter() - t0
                    times[t].append(dt)
                    t_step += dt
                runs.append(t_step)
                total += t_step
            per_row.append(float(np.median(runs)))
            del data
    return {
        "value": round(rows / sum(per_row), 4),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"one whole decode step (step {step}, all {len(tiers)} layers in order: "
                   f"{sum(t == 'full' for t in tiers)} full, {sum(t == 'delta' for t in tiers)} delta, "
                   f"{sum(t == 'sparse' for t in tiers)} sparse) of batch rows 0..{rows - 1} at full context, "
                   f"each tier's layers on that tier's first layer's inputs, median of {repeats} runs per row "
                   f"({total:.1f} s of oracle time in all); tokens/s = rows / sum of the rows' step times "
                   f"(rows are independent)"),
        "seconds_per_layer": {t: round(float(np.median(v)), 4) for t, v in times.items()},
        "oracle_seconds": round(total, 2),
        "repeats": repeats,
        "cpu": cpu_model(),
    }


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else what platform reports."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


if __name__ == "__main__":
    main()
