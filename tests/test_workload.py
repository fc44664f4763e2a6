"""Pins for the shared seeded input generator (host side)."""
import numpy as np
import pytest
import torch

from workload import philox as px
from workload import recipe_for, WORKLOADS as W


def _hex(words):
    return ["%08x" % int(w) for w in words]


# Known-answer vectors published with the Random123 library (Salmon et al., SC'11)
# for Philox4x32 with 10 rounds: (counter words, key words) -> output words.
KAT = [
    ((0, 0, 0, 0), (0, 0), ("6627e8d5", "e169c58d", "bc57ac4c", "9b00dbd8")),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, ("408f276d", "41c83b0e", "a20bc7c6", "6d5451fd")),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     ("d16cfe09", "94fdcceb", "5001e420", "24126ea1")),
]


@pytest.mark.parametrize("ctr,key,expect", KAT)
def test_philox_known_answers(ctr, key, expect):
    out = px.philox4x32_10(*[np.uint64(c) for c in ctr], key[0], key[1])
    assert _hex(out) == list(expect)


def test_normals_moments_and_addressing():
    z = px.normals(7, px.KIND_K, 3, 5, 0, 400_000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    # element addressing: a window equals the slice of a longer draw
    w = px.normals(7, px.KIND_K, 3, 5, 13, 101)
    assert np.array_equal(w, z[13:114])
    rows = px.normals(7, px.KIND_K, 3, np.array([5, 6]), 0, 64)
    assert np.array_equal(rows[0], z[:64])
    assert not np.array_equal(rows[1], z[:64])


def test_bf16_rounding_matches_torch():
    x = px.f32_round(px.normals(1, px.KIND_V, 0, 0, 0, 100_000) * 37.0)
    ours = px.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_recipe_structure_single_layer_8k():
    r = recipe_for("layer1_bf16_b1_t8k")
    wl = r.wl
    T = wl.context
    sal = r.salient_slots(0, 1, 0)
    assert len(sal) == wl.n_salient == len(set(sal))
    assert max(sal) < T - wl.recency * wl.page
    K = r.k_rows(0, 0, 1, 0, T)
    w = r.direction(0, 0, 1)
    assert abs(np.linalg.norm(w.astype(np.float64)) - 1.0) < 1e-6
    proj = K @ w
    # salient keys carry 4 w, the rest are noise
    assert np.all(proj[sal] > 2.0)
    mask = np.ones(T, bool)
    mask[sal] = False
    assert abs(proj[mask].mean()) < 0.1
    # values are bf16-representable
    assert np.array_equal(px.bf16_round(K.astype(np.float32)).astype(np.float64), K)


def test_recipe_drift_moves_ten_percent():
    r = recipe_for("stack28_b8_t16k")
    moves = r.drift_moves(1)
    wl = r.wl
    assert len(moves) == wl.batch * wl.hkv * wl.drift_count
    for b, g, old, new in moves[:8]:
        assert old in r.salient_slots(b, g, 0) and new in r.salient_slots(b, g, 1)
        assert new < wl.context + wl.drift_every - wl.recency * wl.page


def test_ragged_lengths_stack36():
    r = recipe_for("stack36_b32_t8k_32k")
    L = r.lengths0()
    assert L.shape == (32,) and L.min() >= 8192 and L.max() <= 32768
    assert len(set(L.tolist())) > 16


def test_config_budgets_match_workload_text():
    # configs 1-4 state budgets in tokens "incl. recency"; top-k = (budget - recency) / P
    a, b, c, d, e = (W[n] for n in ("layer1_f32_b1_t1k", "layer1_bf16_b1_t8k", "stack28_b8_t16k",
                                     "stack28_b16_t64k", "stack36_b32_t8k_32k"))
    assert b.k_top * 16 == 1536 and b.recency * 16 == 512
    assert (c.k_top + c.recency) * 16 == 2048
    assert (d.k_top + d.recency) * 16 == 4096 and d.recency * 16 == 1024
    assert (e.k_top + e.recency) * 32 == 4096 and e.recency * 32 == 1024
    assert a.k_top == 8 and a.recency * 16 == 64
