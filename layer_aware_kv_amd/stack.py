"""Decode-step driver over a layer stack (the three-tier schedule of DELTA).

"Methodology in Plain English" (DELTA AI summary page): the first two layers and a
few delta-layers attend to the whole context, the delta-layers renewing the page
choice; the other layers attend to the most recent choice, which is renewed for
every generated token.  "Main Findings": the first delta-layer is layer 2 in every
model.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L
from .cache import PagedKVCache, _AGG, _SCOPE, _stream


def layer_tiers(num_layers, full_layers, delta_layers):
    tiers = []
    for layer in range(num_layers):
        if layer in full_layers:
            tiers.append("full")
        elif layer in delta_layers:
            tiers.append("delta")
        else:
            tiers.append("sparse")
    return tiers


class DeltaStack:
    """Runs decode steps of an attention-only stack on one PagedKVCache.

    Per layer and step: append the step's K/V, then full / delta-select / sparse
    attention.  Outputs of every layer are kept in ``out[l]`` / ``lse[l]``; the
    selection installed by delta-layer l in ``sel[l]`` / ``sel_count[l]``.
    """

    def __init__(self, cache: PagedKVCache, tiers, k_top, recency, sm_scale, agg="max", scope="group",
                 fused_append=True, native=True):
        if tiers and tiers[0] == "sparse":
            raise ValueError("a stack cannot start with a sparse layer")
        first_delta = next((i for i, t in enumerate(tiers) if t == "delta"), None)
        if any(t == "sparse" for t in tiers) and (first_delta is None or
                                                  tiers.index("sparse") < first_delta):
            raise ValueError("a sparse layer comes before any delta-layer")
        self.c = cache
        self.tiers = list(tiers)
        self.k_top, self.recency, self.sm_scale = k_top, recency, sm_scale
        self.agg, self.scope = agg, scope
        self.fused_append = fused_append  # append inside the attention call (one launch fewer)
        B, L = cache.max_batch, len(tiers)
        dev = cache.device
        self.out = torch.zeros((L, B, cache.hq, cache.d), dtype=cache.torch_dtype, device=dev)
        self.lse = torch.zeros((L, B, cache.hq), dtype=torch.float32, device=dev)
        R = cache.sel_rows(scope)
        self.sel = {l: torch.full((B, R, k_top + recency), -1, dtype=torch.int32, device=dev)
                    for l, t in enumerate(tiers) if t == "delta"}
        self.sel_count = {l: torch.zeros((B, R), dtype=torch.int32, device=dev)
                          for l, t in enumerate(tiers) if t == "delta"}
        # native path: the whole step is one lak_stack_step call (schedule in C++)
        self.native = native
        self._desc = None

    def _native_desc(self):
        c, L_ = self.c, len(self.tiers)
        B = c.batch
        codes = {"full": 0, "delta": 1, "sparse": 2}
        arr = lambda vals: (C.c_void_p * L_)(*vals)
        d = L.StackStepDesc()
        d.num_layers = L_
        self._tiers = (C.c_int32 * L_)(*[codes[t] for t in self.tiers])
        self._q, self._kn, self._vn = arr([None] * L_), arr([None] * L_), arr([None] * L_)
        self._out = arr([self.out[l, :B].data_ptr() for l in range(L_)])
        self._lse = arr([self.lse[l, :B].data_ptr() for l in range(L_)])
        self._sel = arr([self.sel[l].data_ptr() if l in self.sel else None for l in range(L_)])
        self._cnt = arr([self.sel_count[l].data_ptr() if l in self.sel else None for l in range(L_)])
        d.tiers = C.cast(self._tiers, C.POINTER(C.c_int32))
        for name, a in (("q", self._q), ("k_new", self._kn), ("v_new", self._vn), ("out", self._out),
                        ("lse", self._lse), ("sel", self._sel), ("sel_count", self._cnt)):
            setattr(d, name, C.cast(a, C.POINTER(C.c_void_p)))
        d.sel_capacity = self.k_top + self.recency
        d.sm_scale = self.sm_scale
        d.k_top, d.recency = self.k_top, self.recency
        d.agg, d.scope = _AGG[self.agg], _SCOPE[self.scope]
        return d

    def step(self, q, k_new, v_new, tracer=None):
        """One decode step.  q [L][B][Hq][D]; k_new, v_new [L][B][Hkv][D] (the cache's activation
        dtype: bfloat16 for bf16 and fp8 pools, float32 for f32 pools).

        ``tracer`` (optional) has ``pair(layer, tier)`` returning a (before, after) pair
        of timing events to attach to that layer's decode kernel (objects whose
        ``cuda_event`` is a HIP event handle: ``_lib.TimingEvent`` or a recorded
        torch.cuda.Event), or None.
        """
        c = self.c
        B = c.batch
        if self.native and self.fused_append:
            if self._desc is None:
                self._desc = self._native_desc()
            d = self._desc
            for l in range(len(self.tiers)):
                self._q[l], self._kn[l], self._vn[l] = q[l].data_ptr(), k_new[l].data_ptr(), v_new[l].data_ptr()
            if tracer is not None:
                n = len(self.tiers)
                evs = [tracer.pair(l, t) for l, t in enumerate(self.tiers)]
                self._tb = (C.c_void_p * n)(*[e[0].cuda_event if e else None for e in evs])
                self._ta = (C.c_void_p * n)(*[e[1].cuda_event if e else None for e in evs])
                d.trace_before = C.cast(self._tb, C.POINTER(C.c_void_p))
                d.trace_after = C.cast(self._ta, C.POINTER(C.c_void_p))
            else:
                d.trace_before = d.trace_after = None
            L.check(L.lib().lak_stack_step(c._h, C.byref(d), C.c_void_p(c.ws.data_ptr()), c.ws.numel(), _stream()),
                    "lak_stack_step")
            return
        c.step_begin()
        cur = None
        for layer, tier in enumerate(self.tiers):
            if self.fused_append:
                kn, vn = k_new[layer], v_new[layer]
            else:
                c.kv_append(layer, k_new[layer], v_new[layer])
                kn = vn = None
            out, lse = self.out[layer, :B], self.lse[layer, :B]
            ev = tracer.pair(layer, tier) if tracer is not None else None
            if ev is not None:
                c.trace_decode(*ev)
            if tier == "full":
                c.attn_full(layer, q[layer], self.sm_scale, out, lse, kn, vn)
            elif tier == "delta":
                sel, cnt = self.sel[layer][:B], self.sel_count[layer][:B]
                c.attn_delta_select(layer, q[layer], self.sm_scale, self.k_top, self.recency, self.agg, self.scope,
                                    out, lse, sel, cnt, k_new=kn, v_new=vn)
                cur = (sel, cnt)
            else:
                c.attn_sparse(layer, q[layer], self.sm_scale, cur[0], cur[1], self.scope, out, lse, kn, vn)
            if ev is not None:
                c.trace_decode()
