"""The five synthetic decode workloads (shapes, layer tiers, budgets, seeds), by name.

Plain data: the sizes of the pages' long reasoning decodes (DELTA paper, "Main
Findings": page budget K and recency window L in pages, page size 16, layers 0
and 1 full, layer 2 the first delta-layer; "Methodology": P = 16), scaled to
Qwen-7B-like (28 query / 4 KV heads, d = 128, 28 layers) and Qwen3-8B-like
(32 / 8, d = 128, 36 layers) attention stacks.  No method arithmetic here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int                  # of every input drawn for the workload
    dtype: str                 # "f32" | "bf16"
    num_layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    page: int
    context: int               # prefilled length (max length when ragged)
    ragged_min: int            # 0: every sequence has ``context`` tokens
    full_layers: tuple
    delta_layers: tuple
    k_top: int                 # top-k pages (recency excluded)
    recency: int               # recency window in pages
    sm_scale: float
    q_mode: str                # "scaled_noise" | "salient"
    n_salient: int = 0
    salient_strength: float = 4.0  # salient key = strength * direction + noise
    drift_every: int = 0       # steps between drift events (0: none)
    drift_frac: float = 0.0
    steps: int = 1             # timed decode steps
    warmup: int = 0
    single_layer: bool = False  # one layer run as full, delta and sparse

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def drift_count(self) -> int:
        return int(round(self.drift_frac * self.n_salient))

    def max_tokens(self) -> int:
        """Largest sequence length reached (prefill + warmup + timed steps)."""
        return self.context + self.warmup + self.steps

    def max_pages_per_seq(self) -> int:
        return -(-self.max_tokens() // self.page)

    def tier(self, layer: int) -> str:
        if layer in self.full_layers:
            return "full"
        if layer in self.delta_layers:
            return "delta"
        return "sparse"


_INV_SQRT128 = 1.0 / math.sqrt(128.0)

_ALL = [
    # fp32 single layer, batch 1, T 1024, 8q/2kv, d 64, P 16; q scaled by 1/sqrt(64),
    # sm_scale 1; top 8 pages + 64-token (4-page) recency window.
    Workload(name="layer1_f32_b1_t1k", seed=1000, dtype="f32", num_layers=1, batch=1, hq=8, hkv=2,
             d=64, page=16, context=1024, ragged_min=0, full_layers=(), delta_layers=(0,),
             k_top=8, recency=4, sm_scale=1.0, q_mode="scaled_noise", single_layer=True),
    # Qwen-7B-like single layer, bf16, T 8192; budget 2048 = 1536 top-k (96 pages) + 512 recency (32).
    Workload(name="layer1_bf16_b1_t8k", seed=1001, dtype="bf16", num_layers=1, batch=1, hq=28,
             hkv=4, d=128, page=16, context=8192, ragged_min=0, full_layers=(), delta_layers=(0,),
             k_top=96, recency=32, sm_scale=_INV_SQRT128, q_mode="salient", n_salient=32,
             single_layer=True),
    # 28-layer stack, batch 8, T 16384, delta {2,9,16,23}, budget 2048 incl. 512 recency,
    # 10% of salient positions drift every 100 steps, 256 decode steps.
    Workload(name="stack28_b8_t16k", seed=1002, dtype="bf16", num_layers=28, batch=8, hq=28, hkv=4,
             d=128, page=16, context=16384, ragged_min=0, full_layers=(0, 1), delta_layers=(2, 9, 16, 23),
             k_top=96, recency=32, sm_scale=_INV_SQRT128, q_mode="salient", n_salient=32,
             drift_every=100, drift_frac=0.1, steps=256, warmup=0),
    # the same stack at long reasoning length: batch 16, T 65536, budget 4096 incl. 1024 recency.
    Workload(name="stack28_b16_t64k", seed=1003, dtype="bf16", num_layers=28, batch=16, hq=28, hkv=4,
             d=128, page=16, context=65536, ragged_min=0, full_layers=(0, 1), delta_layers=(2, 9, 16, 23),
             k_top=192, recency=64, sm_scale=_INV_SQRT128, q_mode="salient", n_salient=32,
             drift_every=100, drift_frac=0.1, steps=32, warmup=4),
    # Qwen3-8B-like 36-layer stack, 32q/8kv, P 32, batch 32, ragged T ~ U[8192, 32768],
    # delta every 8 layers from layer 2, budget 4096 incl. 1024 recency (96 + 32 pages of 32).
    Workload(name="stack36_b32_t8k_32k", seed=1004, dtype="bf16", num_layers=36, batch=32, hq=32,
             hkv=8, d=128, page=32, context=32768, ragged_min=8192, full_layers=(0, 1),
             delta_layers=(2, 10, 18, 26, 34), k_top=96, recency=32, sm_scale=_INV_SQRT128,
             q_mode="salient", n_salient=32, steps=32, warmup=4),
]

WORKLOADS = {w.name: w for w in _ALL}
STACKS = [w.name for w in _ALL if not w.single_layer]  # the layer-stack workloads, smallest first


def get(name: str) -> Workload:
    return WORKLOADS[name]
