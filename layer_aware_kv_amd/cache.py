"""Python binding of the paged KV cache and the decode-attention calls.

Argument marshalling only: tensors are passed to the C ABI as device pointers
together with torch's current HIP stream; every step runs in the library's
kernels.  PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L

# activations (q, out, k_new / v_new, prefill rows) per cache dtype; fp8 pools take bfloat16 rows
_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.bfloat16}
_LAK_DT = {"bf16": L.LAK_BF16, "f32": L.LAK_F32, "fp8": L.LAK_FP8_E4M3}
_POOL_DT = {"bf16": (torch.bfloat16, 2), "f32": (torch.float32, 4), "fp8": (torch.uint8, 1)}
_AGG = {"max": L.LAK_AGG_MAX, "sum": L.LAK_AGG_SUM}
_SCOPE = {"group": L.LAK_SCOPE_GROUP, "all": L.LAK_SCOPE_ALL}


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class PagedKVCache:
    """One paged GQA KV cache shared by all layers (one K and one V pool per layer).

    Pools hold ``num_pages`` pages of [Hkv][P][D] elements each (``dtype`` "bf16",
    "f32", or "fp8": E4M3 codes plus a float32 scale per token row); the page table and
    sequence lengths live in device memory and are maintained by the library.  q, out,
    k_new / v_new and prefill rows use ``torch_dtype`` (bfloat16 for an fp8 cache).
    """

    def __init__(self, num_layers, max_batch, num_q_heads, num_kv_heads, head_dim, page_size,
                 max_pages_per_seq, num_pages, dtype="bf16", device="cuda"):
        self.num_layers = num_layers
        self.max_batch = max_batch
        self.hq = num_q_heads
        self.hkv = num_kv_heads
        self.d = head_dim
        self.page = page_size
        self.max_pages = max_pages_per_seq
        self.num_pages = num_pages
        self.dtype = dtype
        self.torch_dtype = _TORCH_DT[dtype]
        self.device = torch.device(device)
        lib = L.lib()
        desc = L.CacheDesc(num_layers, max_batch, num_q_heads, num_kv_heads, head_dim, page_size,
                           max_pages_per_seq, _LAK_DT[dtype], num_pages, None, None, None, None)
        pool_bytes = lib.lak_pool_bytes(C.byref(desc))
        if pool_bytes <= 0:
            raise L.LakError(L.LAK_EINVAL, "lak_pool_bytes", "invalid description")
        pdt, esz = _POOL_DT[dtype]
        elems = pool_bytes // esz
        self.k_pools = [torch.empty(elems, dtype=pdt, device=self.device) for _ in range(num_layers)]
        self.v_pools = [torch.empty(elems, dtype=pdt, device=self.device) for _ in range(num_layers)]
        self.page_table = torch.zeros((max_batch, max_pages_per_seq), dtype=torch.int32, device=self.device)
        self.seq_lens = torch.zeros(max_batch, dtype=torch.int32, device=self.device)
        kp = (C.c_void_p * num_layers)(*[t.data_ptr() for t in self.k_pools])
        vp = (C.c_void_p * num_layers)(*[t.data_ptr() for t in self.v_pools])
        desc.k_pools = C.cast(kp, C.POINTER(C.c_void_p))
        desc.v_pools = C.cast(vp, C.POINTER(C.c_void_p))
        desc.page_table = self.page_table.data_ptr()
        desc.seq_lens = self.seq_lens.data_ptr()
        h = C.c_void_p()
        L.check(lib.lak_cache_create(C.byref(desc), C.byref(h)), "lak_cache_create")
        self._h = h
        self.ws = torch.empty(lib.lak_workspace_bytes(h), dtype=torch.uint8, device=self.device)
        self.batch = 0

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and L._lib is not None:
            L._lib.lak_cache_destroy(h)
            self._h = None

    # ------------------------------------------------------------ metadata
    def seq_reset(self, lengths, reserve_tokens=0):
        lens = [int(x) for x in lengths]
        arr = (C.c_int32 * max(1, len(lens)))(*lens)
        L.check(L.lib().lak_seq_reset(self._h, len(lens), arr, int(reserve_tokens), _stream()), "lak_seq_reset")
        self.batch = len(lens)

    def step_begin(self):
        L.check(L.lib().lak_step_begin(self._h, _stream()), "lak_step_begin")

    def seq_lens_host(self):
        out = (C.c_int32 * max(1, self.max_batch))()
        n = C.c_int32()
        L.check(L.lib().lak_seq_lens_host(self._h, out, self.max_batch, C.byref(n)), "lak_seq_lens_host")
        return [out[i] for i in range(max(n.value, 0))]

    def page_table_host(self, b):
        out = (C.c_int32 * self.max_pages)()
        n = C.c_int32()
        L.check(L.lib().lak_page_table_host(self._h, b, out, self.max_pages, C.byref(n)), "lak_page_table_host")
        return [out[i] for i in range(n.value)]

    def free_pages(self):
        return L.lib().lak_free_pages(self._h)

    def trace_decode(self, before=None, after=None):
        """Record torch.cuda.Event ``before`` / ``after`` around the decode kernel of
        the following attention calls (None, None stops).  The events must already
        exist on the device (torch creates one at its first ``record()``)."""
        if before is not None and (before.cuda_event == 0 or after.cuda_event == 0):
            raise ValueError("trace events not created yet: record() each once first")
        b = None if before is None else C.c_void_p(before.cuda_event)
        a = None if after is None else C.c_void_p(after.cuda_event)
        L.check(L.lib().lak_trace_decode(self._h, b, a), "lak_trace_decode")

    # ------------------------------------------------------------ KV writes
    def kv_append(self, layer, k_new, v_new):
        L.check(L.lib().lak_kv_append(self._h, layer, _ptr(k_new), _ptr(v_new), _stream()), "lak_kv_append")

    def kv_prefill(self, layer, k, v):
        """k, v: [B][Hkv][t_stride][D] contiguous, in the activation dtype (bfloat16 rows are
        encoded for an fp8 cache)."""
        L.check(L.lib().lak_kv_prefill(self._h, layer, _ptr(k), _ptr(v), k.shape[2], _stream()), "lak_kv_prefill")

    def kv_write_rows(self, layer, rows, k_rows, v_rows=None):
        L.check(L.lib().lak_kv_write_rows(self._h, layer, rows.shape[0], _ptr(rows), _ptr(k_rows), _ptr(v_rows),
                                          _stream()), "lak_kv_write_rows")

    def kv_gather(self, layer, b, g, t0, n):
        """Rows [t0, t0+n) of (b, g) in the pool's element type (uint8 E4M3 codes for fp8)."""
        pdt = _POOL_DT[self.dtype][0]
        k = torch.empty((n, self.d), dtype=pdt, device=self.device)
        v = torch.empty((n, self.d), dtype=pdt, device=self.device)
        L.check(L.lib().lak_kv_gather(self._h, layer, b, g, t0, n, _ptr(k), _ptr(v), _stream()), "lak_kv_gather")
        return k, v

    def kv_gather_scales(self, layer, b, g, t0, n):
        """fp8 caches: the float32 scales of rows [t0, t0+n) of (b, g)."""
        k = torch.empty(n, dtype=torch.float32, device=self.device)
        v = torch.empty(n, dtype=torch.float32, device=self.device)
        L.check(L.lib().lak_kv_gather_scales(self._h, layer, b, g, t0, n, _ptr(k), _ptr(v), _stream()),
                "lak_kv_gather_scales")
        return k, v

    # ------------------------------------------------------------ attention
    def _out(self, out, lse):
        if out is None:
            out = torch.empty((self.batch, self.hq, self.d), dtype=self.torch_dtype, device=self.device)
        if lse is None:
            lse = torch.empty((self.batch, self.hq), dtype=torch.float32, device=self.device)
        return out, lse

    def attn_full(self, layer, q, sm_scale, out=None, lse=None, k_new=None, v_new=None):
        """Full attention; with k_new / v_new the call also appends this step's token."""
        out, lse = self._out(out, lse)
        L.check(L.lib().lak_attn_full(self._h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                      _ptr(out), _ptr(lse), _ptr(self.ws), self.ws.numel(), _stream()),
                "lak_attn_full")
        return out, lse

    def sel_rows(self, scope):
        return self.hkv if scope == "group" else 1

    def attn_delta_select(self, layer, q, sm_scale, k_top, recency, agg="max", scope="group", out=None,
                          lse=None, sel=None, sel_count=None, page_scores=None, sel_capacity=None, k_new=None,
                          v_new=None):
        out, lse = self._out(out, lse)
        R = self.sel_rows(scope)
        cap = sel_capacity or (k_top + recency)
        if sel is None:
            sel = torch.empty((self.batch, R, cap), dtype=torch.int32, device=self.device)
        if sel_count is None:
            sel_count = torch.empty((self.batch, R), dtype=torch.int32, device=self.device)
        L.check(L.lib().lak_attn_delta_select(
            self._h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale), _ptr(out), _ptr(lse), int(k_top),
            int(recency), _AGG[agg],
            _SCOPE[scope], _ptr(sel), _ptr(sel_count), sel.shape[-1], _ptr(page_scores), _ptr(self.ws),
            self.ws.numel(), _stream()), "lak_attn_delta_select")
        return out, lse, sel, sel_count

    def page_select(self, page_scores, k_top, recency, scope="group", sel=None, sel_count=None):
        R = self.sel_rows(scope)
        if sel is None:
            sel = torch.empty((self.batch, R, k_top + recency), dtype=torch.int32, device=self.device)
        if sel_count is None:
            sel_count = torch.empty((self.batch, R), dtype=torch.int32, device=self.device)
        L.check(L.lib().lak_page_select(self._h, _ptr(page_scores), _SCOPE[scope], int(k_top), int(recency),
                                        _ptr(sel), _ptr(sel_count), sel.shape[-1], _stream()), "lak_page_select")
        return sel, sel_count

    def attn_sparse(self, layer, q, sm_scale, sel, sel_count, scope="group", out=None, lse=None, k_new=None,
                    v_new=None):
        out, lse = self._out(out, lse)
        L.check(L.lib().lak_attn_sparse(self._h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                        _ptr(sel), _ptr(sel_count), sel.shape[-1], _SCOPE[scope], _ptr(out),
                                        _ptr(lse), _ptr(self.ws), self.ws.numel(), _stream()), "lak_attn_sparse")
        return out, lse

    def attn_sparse_noalloc(self, layer, q, sm_scale, sel, sel_count, scope="group", out=None, lse=None,
                            k_new=None, v_new=None):
        """attn_sparse with its split partials in the library's static device scratch
        instead of the workspace (for callers that cannot allocate; calls that overlap on
        the device race).  ``out`` / ``lse`` must be given where the caller cannot allocate."""
        out, lse = self._out(out, lse)
        L.check(L.lib().lak_attn_sparse_noalloc(self._h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                                _ptr(sel), _ptr(sel_count), sel.shape[-1], _SCOPE[scope], _ptr(out),
                                                _ptr(lse), _stream()), "lak_attn_sparse_noalloc")
        return out, lse
