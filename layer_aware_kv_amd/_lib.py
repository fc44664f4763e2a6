"""ctypes view of liblak.so (the C ABI declared in include/lak.h)."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblak.so")

LAK_OK, LAK_EINVAL, LAK_ENOPAGE, LAK_EHIP, LAK_EUNSUPPORTED, LAK_ESTATE = 0, -1, -2, -3, -4, -5
LAK_BF16, LAK_F32, LAK_FP8_E4M3 = 0, 1, 2
LAK_AGG_MAX, LAK_AGG_SUM = 0, 1
LAK_SCOPE_GROUP, LAK_SCOPE_ALL = 0, 1

STATUS_NAMES = {0: "LAK_OK", -1: "LAK_EINVAL", -2: "LAK_ENOPAGE", -3: "LAK_EHIP", -4: "LAK_EUNSUPPORTED",
                -5: "LAK_ESTATE"}


class LakError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class CacheDesc(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("max_batch", C.c_int32), ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page_size", C.c_int32),
        ("max_pages_per_seq", C.c_int32), ("dtype", C.c_int32), ("num_pages", C.c_int64),
        ("k_pools", C.POINTER(C.c_void_p)), ("v_pools", C.POINTER(C.c_void_p)),
        ("page_table", C.c_void_p), ("seq_lens", C.c_void_p),
    ]


class StackStepDesc(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("tiers", C.POINTER(C.c_int32)),
        ("q", C.POINTER(C.c_void_p)), ("k_new", C.POINTER(C.c_void_p)), ("v_new", C.POINTER(C.c_void_p)),
        ("out", C.POINTER(C.c_void_p)), ("lse", C.POINTER(C.c_void_p)),
        ("sel", C.POINTER(C.c_void_p)), ("sel_count", C.POINTER(C.c_void_p)),
        ("sel_capacity", C.c_int32), ("sm_scale", C.c_float),
        ("k_top", C.c_int32), ("recency", C.c_int32), ("agg", C.c_int32), ("scope", C.c_int32),
        ("trace_before", C.POINTER(C.c_void_p)), ("trace_after", C.POINTER(C.c_void_p)),
    ]


_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64
_F = C.c_float
_S = C.c_int  # lak_status

# name -> (restype, argtypes); every symbol include/lak.h declares
SIGNATURES = {
    "lak_pool_bytes": (_I64, [C.POINTER(CacheDesc)]),
    "lak_cache_create": (_S, [C.POINTER(CacheDesc), C.POINTER(_P)]),
    "lak_cache_destroy": (_S, [_P]),
    "lak_seq_reset": (_S, [_P, _I32, C.POINTER(_I32), _I32, _P]),
    "lak_step_begin": (_S, [_P, _P]),
    "lak_seq_lens_host": (_S, [_P, C.POINTER(_I32), _I32, C.POINTER(_I32)]),
    "lak_page_table_host": (_S, [_P, _I32, C.POINTER(_I32), _I32, C.POINTER(_I32)]),
    "lak_free_pages": (_I64, [_P]),
    "lak_workspace_bytes": (C.c_size_t, [_P]),
    "lak_kv_append": (_S, [_P, _I32, _P, _P, _P]),
    "lak_kv_prefill": (_S, [_P, _I32, _P, _P, _I64, _P]),
    "lak_kv_write_rows": (_S, [_P, _I32, _I32, _P, _P, _P, _P]),
    "lak_kv_gather": (_S, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "lak_kv_gather_scales": (_S, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "lak_attn_full": (_S, [_P, _I32, _P, _P, _P, _F, _P, _P, _P, C.c_size_t, _P]),
    "lak_attn_delta_select": (_S, [_P, _I32, _P, _P, _P, _F, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _I32, _P,
                                   _P, C.c_size_t, _P]),
    "lak_page_select": (_S, [_P, _P, _I32, _I32, _I32, _P, _P, _I32, _P]),
    "lak_attn_sparse": (_S, [_P, _I32, _P, _P, _P, _F, _P, _P, _I32, _I32, _P, _P, _P, C.c_size_t, _P]),
    "lak_attn_sparse_noalloc": (_S, [_P, _I32, _P, _P, _P, _F, _P, _P, _I32, _I32, _P, _P, _P]),
    "lak_stack_step": (_S, [_P, C.POINTER(StackStepDesc), _P, C.c_size_t, _P]),
    "lak_trace_decode": (_S, [_P, _P, _P]),
    "lak_last_error": (C.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library; raises if the HIP build is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m layer_aware_kv_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


_hip = None
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip_lib():
    global _hip
    if _hip is None:
        h = C.CDLL("libamdhip64.so")
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        h.hipEventElapsedTime.restype = C.c_int
        h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        h.hipEventCreateWithFlags.restype = C.c_int
        h.hipEventDestroy.argtypes = [C.c_void_p]
        h.hipEventDestroy.restype = C.c_int
        _hip = h
    return _hip


def event_elapsed_ms(before, after) -> float:
    """hipEventElapsedTime of two completed events (TimingEvent, or torch.cuda.Event
    objects recorded by the library, which torch itself does not know were recorded)."""
    ms = C.c_float()
    rc = _hip_lib().hipEventElapsedTime(C.byref(ms), C.c_void_p(before.cuda_event), C.c_void_p(after.cuda_event))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed with hipError {rc}")
    return ms.value


class TimingEvent:
    """A HIP event for timing kernels only, on the current device: created with
    hipEventDisableSystemFence, so that recording it (the library attaches it to a decode
    kernel's dispatch) adds no system-scope cache writeback and invalidation to the stream
    -- with the default flags each attached pair costs the stream a few microseconds.  Its
    time is read (event_elapsed_ms) only after the device has been synchronised.  Exposes
    the handle as ``cuda_event``, like torch.cuda.Event."""

    def __init__(self):
        h = C.c_void_p()
        rc = _hip_lib().hipEventCreateWithFlags(C.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0 or not h.value:
            raise RuntimeError(f"hipEventCreateWithFlags failed with hipError {rc}")
        self.cuda_event = h.value

    def __del__(self):
        if getattr(self, "cuda_event", 0) and _hip is not None:
            _hip.hipEventDestroy(C.c_void_p(self.cuda_event))
            self.cuda_event = 0


def check(status: int, where: str):
    if status != LAK_OK:
        raise LakError(status, where, lib().lak_last_error().decode())
