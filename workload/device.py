"""Device-side fill of the synthetic inputs (libworkload.so), element-for-element equal
to ``recipe.Recipe`` on the host.  Plain input generation: no attention arithmetic."""
from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np
import torch

from . import philox as px
from .recipe import Recipe

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libworkload.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m layer_aware_kv_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I, I64, U64, F = C.c_void_p, C.c_int, C.c_int64, C.c_uint64, C.c_float
        L.wl_fill_tokens.argtypes = [P, I, I64, I64, I, P, I64, I, I, U64, I64, I64, I, F, F, P, I, P]
        L.wl_apply_salient.argtypes = [P, I, I64, I, I, P, P, I64, I64, I64, I64, I, I, U64, C.c_float, P]
        L.wl_fill_rows.argtypes = [P, I, I, I, P, P, P, P, I, I, U64, C.c_float, P]
        for f in (L.wl_fill_tokens, L.wl_apply_salient, L.wl_fill_rows):
            f.restype = I
        _lib = L
    return _lib


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _st():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _chk(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


class DeviceInputs:
    """Fills device tensors with the recipe's values."""

    def __init__(self, recipe: Recipe, device="cuda"):
        self.r = recipe
        self.wl = recipe.wl
        self.device = torch.device(device)
        self.dt = 0 if self.wl.dtype == "bf16" else 1
        self.torch_dtype = torch.bfloat16 if self.wl.dtype == "bf16" else torch.float32
        self._dirs = {}

    def dirs(self, layer):
        if layer not in self._dirs:
            self._dirs[layer] = torch.from_numpy(self.r.directions(layer)).to(self.device)
        return self._dirs[layer]

    def salient_positions(self, epoch):
        wl = self.wl
        if wl.n_salient == 0:
            return None
        pos = np.array([self.r.salient_slots(b, g, epoch) for b in range(wl.batch) for g in range(wl.hkv)],
                       dtype=np.int32)
        return torch.from_numpy(pos).to(self.device)

    def fill_kv(self, layer, k_out, v_out, t_stride, epoch=0, sal=None):
        """Logical K, V of all sequences, positions [0, t_stride): [B][Hkv][t_stride][D]."""
        wl = self.wl
        R = wl.batch * wl.hkv
        for kind, out in ((px.KIND_K, k_out), (px.KIND_V, v_out)):
            _chk(lib().wl_fill_tokens(_p(out), self.dt, R, t_stride, wl.d, None, 0, kind, layer, self.r.seed,
                                      t_stride * wl.d, wl.d, 0, 0.0, 0.0, None, 1, _st()), "wl_fill_tokens")
        if wl.n_salient:
            pos = self.salient_positions(epoch) if sal is None else sal
            _chk(lib().wl_apply_salient(_p(k_out), self.dt, R, wl.n_salient, wl.d, _p(pos), _p(self.dirs(layer)),
                                        0, t_stride, t_stride * wl.d, wl.d, px.KIND_K, layer, self.r.seed,
                                        float(wl.salient_strength), _st()),
                 "wl_apply_salient")

    def fill_queries(self, layer, step0, n_steps, out):
        """Queries of steps [step0, step0 + n_steps): out [n_steps][B][Hq][D]."""
        wl = self.wl
        R = wl.batch * wl.hq
        if wl.q_mode == "scaled_noise":
            mode, c1, c2, dirs = 1, 1.0 / math.sqrt(wl.d), 0.0, None
        else:
            mode, c1, c2, dirs = 2, float(self.r.c1), float(self.r.c2), self.dirs(layer)
        _chk(lib().wl_fill_tokens(_p(out), self.dt, R, n_steps, wl.d, None, step0, px.KIND_Q, layer, self.r.seed,
                                  wl.d, R * wl.d, mode, c1, c2, _p(dirs), wl.group, _st()), "wl_fill_tokens(q)")

    def fill_new_kv(self, layer, step0, n_steps, k_out, v_out):
        """Appended token of each step: position T0_b + s.  k_out, v_out [n_steps][B][Hkv][D]."""
        wl = self.wl
        R = wl.batch * wl.hkv
        t0 = np.repeat(self.r.lengths0() + step0, wl.hkv).astype(np.int32)
        t0_dev = torch.from_numpy(t0).to(self.device)
        for kind, out in ((px.KIND_K, k_out), (px.KIND_V, v_out)):
            _chk(lib().wl_fill_tokens(_p(out), self.dt, R, n_steps, wl.d, _p(t0_dev), 0, kind, layer, self.r.seed,
                                      wl.d, R * wl.d, 0, 0.0, 0.0, None, 1, _st()), "wl_fill_tokens(new)")

    def drift_rows(self, layer, epoch):
        """Rows that the drift event starting ``epoch`` rewrites: (rows [n][3] int32, k_rows [n][D])."""
        wl = self.wl
        moves = self.r.drift_moves(epoch)
        if not moves:
            return None, None
        rows, srow, toks, sal = [], [], [], []
        for b, g, old, new in moves:
            rows += [(b, g, old), (b, g, new)]
            srow += [b * wl.hkv + g] * 2
            toks += [old, new]
            sal += [0, 1]
        n = len(rows)
        rows_t = torch.tensor(rows, dtype=torch.int32, device=self.device)
        srow_t = torch.tensor(srow, dtype=torch.int32, device=self.device)
        toks_t = torch.tensor(toks, dtype=torch.int32, device=self.device)
        sal_t = torch.tensor(sal, dtype=torch.int32, device=self.device)
        dirs = self.dirs(layer)[srow_t.long()].contiguous()
        k_rows = torch.empty((n, wl.d), dtype=self.torch_dtype, device=self.device)
        _chk(lib().wl_fill_rows(_p(k_rows), self.dt, n, wl.d, _p(srow_t), _p(toks_t), _p(dirs), _p(sal_t),
                                px.KIND_K, layer, self.r.seed, float(wl.salient_strength), _st()), "wl_fill_rows")
        return rows_t, k_rows
