"""Small seeded test cases: N(0,1) queries / keys / values of a given shape, rounded
to the stored dtype, drawn from the same counter-based generator.  Input data only."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox as px


@dataclass
class Case:
    dtype: str
    q: np.ndarray        # [B][Hq][D] float64 (values exact in dtype)
    K: np.ndarray        # [B][Hkv][Tmax][D]
    V: np.ndarray
    lengths: list
    k_new: np.ndarray = None   # [B][Hkv][D] token appended by a decode step
    v_new: np.ndarray = None


def random_case(seed: int, batch: int, hq: int, hkv: int, d: int, lengths, dtype: str = "bf16",
                q_scale: float = 1.0, k_scale: float = 1.0) -> Case:
    """``q_scale`` / ``k_scale`` must be powers of two so that scaling stays exact."""
    lengths = [int(x) for x in lengths]
    tmax = max(max(lengths), 1)

    def draw(kind, rows, count):
        return px.normals(seed, kind, 0, np.arange(rows), 0, count)

    q = px.to_dtype_values(draw(px.KIND_Q, batch * hq, d) * q_scale, dtype).reshape(batch, hq, d)
    K = px.to_dtype_values(draw(px.KIND_K, batch * hkv, tmax * d) * k_scale, dtype).reshape(batch, hkv, tmax, d)
    V = px.to_dtype_values(draw(px.KIND_V, batch * hkv, tmax * d), dtype).reshape(batch, hkv, tmax, d)
    kn = px.to_dtype_values(px.normals(seed, px.KIND_K, 1, np.arange(batch * hkv), 0, d) * k_scale, dtype)
    vn = px.to_dtype_values(px.normals(seed, px.KIND_V, 1, np.arange(batch * hkv), 0, d), dtype)
    return Case(dtype, q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), lengths,
                kn.reshape(batch, hkv, d).astype(np.float64), vn.reshape(batch, hkv, d).astype(np.float64))


def plant_salient(case: Case, b: int, g: int, positions, head_group: int, strength: float = 4.0):
    """Make keys at ``positions`` of (b, g) point along the group's first query
    (a sharp far-token attention target); values stay exact in the dtype."""
    qv = case.q[b, g * head_group]
    w = qv / np.linalg.norm(qv)
    for t in positions:
        k = px.to_dtype_values(strength * w + case.K[b, g, t], case.dtype)
        case.K[b, g, t] = k
    return case
