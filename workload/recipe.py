"""Host-side materialisation of the synthetic decode inputs.

Every input is a pure function of (workload, seed, layer, batch row, head,
position, step), drawn from ``philox.normals``; the device fill kernels in
``workload/csrc/fill.hip`` compute the same values.  Definitions:

* prefilled length T0_b: ``context`` (or, ragged, ``ragged_min + w mod
  (context - ragged_min + 1)`` for the b-th raw word of the KIND_LEN stream);
* K[l,b,g,t,:] = noise_K(t) (+ s w_{l,b,g}, s = salient_strength (4 by default), when t is a salient position of the
  current drift epoch), V[l,b,g,t,:] = noise_V(t), rounded to the stored dtype;
  the token appended at decode step s sits at position T0_b + s and is plain noise;
* salient direction w_{l,b,g} = n / |n| for n ~ N(0, I_D) (KIND_DIR), float32;
* q: "scaled_noise" -> z / 8 (d = 64, an exact power-of-two scale);
  "salient" -> q_h = f32(c1 * w_{g(h)}) + f32(c2 * z_h) with c1 = 0.9 sqrt(D),
  c2 = sqrt(0.19), each product and the sum rounded to float32;
* salient positions (epoch 0): ``n_salient`` distinct positions drawn in
  [0, T0_b - recency*P) from the KIND_POS stream (position = word mod range,
  duplicates skipped, in draw order); at drift epoch e >= 1 (before step
  e*drift_every) slots (e-1)*m .. (e-1)*m+m-1 (mod n_salient), m = drift_count,
  move to new distinct positions in [0, T0_b + e*drift_every - recency*P).

Nothing here computes attention, scores or selections.
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

from . import philox as px
from .configs import Workload


class Recipe:
    def __init__(self, wl: Workload):
        self.wl = wl
        self.seed = wl.seed
        self.c1 = np.float32(0.9 * math.sqrt(wl.d))
        self.c2 = np.float32(math.sqrt(0.19))
        self._pos_cache = {}

    # ----------------------------------------------------------------- lengths
    def lengths0(self) -> np.ndarray:
        wl = self.wl
        if wl.ragged_min <= 0:
            return np.full(wl.batch, wl.context, dtype=np.int64)
        span = wl.context - wl.ragged_min + 1
        words = px.raw_words(self.seed, px.KIND_LEN, 0, 0, -(-wl.batch // 4)).reshape(-1)[: wl.batch]
        return wl.ragged_min + (words.astype(np.int64) % span)

    def length_at(self, b: int, step: int) -> int:
        """Sequence length during decode step ``step`` (after that step's append)."""
        return int(self.lengths0()[b]) + step + 1

    # -------------------------------------------------------------- directions
    def direction(self, layer: int, b: int, g: int) -> np.ndarray:
        wl = self.wl
        n = px.normals(self.seed, px.KIND_DIR, layer, b * wl.hkv + g, 0, wl.d)
        return px.f32_round(n / np.sqrt(np.dot(n, n)))

    def directions(self, layer: int) -> np.ndarray:
        """[B*Hkv, D] float32 unit directions of one layer."""
        wl = self.wl
        rows = np.arange(wl.batch * wl.hkv)
        n = px.normals(self.seed, px.KIND_DIR, layer, rows, 0, wl.d)
        return px.f32_round(n / np.sqrt(np.sum(n * n, axis=1, keepdims=True)))

    # --------------------------------------------------------- salient sets
    def _draw_distinct(self, row: int, epoch: int, lo_excl: set, count: int, hi: int) -> list:
        out = []
        taken = set(lo_excl)
        block = 0
        while len(out) < count:
            words = px.raw_words(self.seed, px.KIND_POS, epoch, row, 64, block0=block).reshape(-1)
            block += 64
            for w in words:
                p = int(w) % hi
                if p not in taken:
                    taken.add(p)
                    out.append(p)
                    if len(out) == count:
                        break
        return out

    def salient_slots(self, b: int, g: int, epoch: int) -> list:
        """Salient positions by slot (list of n_salient ints) at a drift epoch."""
        wl = self.wl
        key = (b, g, epoch)
        if key in self._pos_cache:
            return self._pos_cache[key]
        if wl.n_salient == 0:
            res = []
        elif epoch == 0:
            hi = int(self.lengths0()[b]) - wl.recency * wl.page
            res = self._draw_distinct(b * wl.hkv + g, 0, set(), wl.n_salient, max(hi, wl.n_salient))
        else:
            prev = list(self.salient_slots(b, g, epoch - 1))
            m = wl.drift_count
            hi = int(self.lengths0()[b]) + epoch * wl.drift_every - wl.recency * wl.page
            new = self._draw_distinct(b * wl.hkv + g, epoch, set(prev), m, hi)
            for i in range(m):
                prev[((epoch - 1) * m + i) % wl.n_salient] = new[i]
            res = prev
        self._pos_cache[key] = res
        return res

    def epoch_of_step(self, step: int) -> int:
        de = self.wl.drift_every
        return step // de if de > 0 else 0

    def drift_moves(self, epoch: int):
        """[(b, g, old_pos, new_pos)] for the drift event that starts ``epoch``."""
        wl = self.wl
        moves = []
        for b in range(wl.batch):
            for g in range(wl.hkv):
                old = self.salient_slots(b, g, epoch - 1)
                new = self.salient_slots(b, g, epoch)
                for s in range(wl.n_salient):
                    if old[s] != new[s]:
                        moves.append((b, g, old[s], new[s]))
        return moves

    # -------------------------------------------------------------- K, V, q
    def k_rows(self, layer: int, b: int, g: int, t0: int, t1: int, epoch: int = 0) -> np.ndarray:
        """Stored K values for positions [t0, t1) as float64 [t1-t0, D]."""
        wl = self.wl
        z = px.normals(self.seed, px.KIND_K, layer, b * wl.hkv + g, t0 * wl.d, (t1 - t0) * wl.d)
        z32 = px.f32_round(z).reshape(t1 - t0, wl.d)
        sal = [p for p in self.salient_slots(b, g, epoch) if t0 <= p < t1]
        if sal:
            w = self.direction(layer, b, g)
            idx = np.asarray(sal) - t0
            z32[idx] = (np.float32(wl.salient_strength) * w)[None, :] + z32[idx]
        if wl.dtype == "bf16":
            z32 = px.bf16_round(z32)
        return z32.astype(np.float64)

    def v_rows(self, layer: int, b: int, g: int, t0: int, t1: int) -> np.ndarray:
        wl = self.wl
        z = px.normals(self.seed, px.KIND_V, layer, b * wl.hkv + g, t0 * wl.d, (t1 - t0) * wl.d)
        return px.to_dtype_values(z, wl.dtype).reshape(t1 - t0, wl.d).astype(np.float64)

    def q(self, layer: int, step: int, b: int) -> np.ndarray:
        """Stored query values [Hq, D] (float64) of decode step ``step``."""
        wl = self.wl
        rows = b * wl.hq + np.arange(wl.hq)
        z = px.normals(self.seed, px.KIND_Q, layer, rows, step * wl.d, wl.d)
        z32 = px.f32_round(z)
        if wl.q_mode == "scaled_noise":
            q32 = z32 * np.float32(1.0 / math.sqrt(wl.d))
        else:
            w = np.stack([self.direction(layer, b, h // wl.group) for h in range(wl.hq)])
            q32 = (self.c1 * w).astype(np.float32) + (self.c2 * z32).astype(np.float32)
        q32 = q32.astype(np.float32)
        if wl.dtype == "bf16":
            q32 = px.bf16_round(q32)
        return q32.astype(np.float64)

    # ------------------------------------------------------------ convenience
    def layer_kv(self, layer: int, b: int, T: int, epoch: int = 0):
        """(K, V) of one batch row as float64 [Hkv, T, D]."""
        wl = self.wl
        K = np.stack([self.k_rows(layer, b, g, 0, T, epoch) for g in range(wl.hkv)])
        V = np.stack([self.v_rows(layer, b, g, 0, T) for g in range(wl.hkv)])
        return K, V


@lru_cache(maxsize=8)
def recipe_for(name: str) -> Recipe:
    from .configs import get
    return Recipe(get(name))
