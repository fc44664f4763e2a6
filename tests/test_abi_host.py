"""CPU tests of the C ABI: exported symbols, argument validation, the host page
allocator (metadata-only cache: no device is touched), and the byte accounting."""
import ctypes as C
import os
import re

import pytest

from layer_aware_kv_amd import _lib as L
from layer_aware_kv_amd import accounting as acc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "lak.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lak_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared_symbols()
    assert len(names) >= 17
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, n
    assert set(L.SIGNATURES) == set(names)


def _desc(num_pages=64, max_batch=4, max_pages=16, page=16, hq=8, hkv=2, d=64, dtype=L.LAK_BF16, layers=2):
    return L.CacheDesc(layers, max_batch, hq, hkv, d, page, max_pages, dtype, num_pages, None, None, None, None)


def _create(**kw):
    h = C.c_void_p()
    st = L.lib().lak_cache_create(C.byref(_desc(**kw)), C.byref(h))
    return st, h


def _lens(h, cap=8):
    out = (C.c_int32 * cap)()
    n = C.c_int32()
    L.check(L.lib().lak_seq_lens_host(h, out, cap, C.byref(n)), "lens")
    return [out[i] for i in range(n.value)]


def _pages(h, b, cap=64):
    out = (C.c_int32 * cap)()
    n = C.c_int32()
    L.check(L.lib().lak_page_table_host(h, b, out, cap, C.byref(n)), "pages")
    return [out[i] for i in range(n.value)]


def test_pool_bytes():
    d = _desc(num_pages=10, hkv=4, page=16, d=128, dtype=L.LAK_BF16)
    assert L.lib().lak_pool_bytes(C.byref(d)) == 10 * 4 * 16 * 128 * 2
    d = _desc(num_pages=3, hkv=2, page=32, d=64, dtype=L.LAK_F32)
    assert L.lib().lak_pool_bytes(C.byref(d)) == 3 * 2 * 32 * 64 * 4
    # fp8: one byte per code plus a float32 scale per (page, kv head, token) row
    d = _desc(num_pages=5, hkv=4, page=16, d=128, dtype=L.LAK_FP8_E4M3)
    assert L.lib().lak_pool_bytes(C.byref(d)) == 5 * 4 * 16 * 128 + 5 * 4 * 16 * 4
    st, h = _create(dtype=L.LAK_FP8_E4M3)
    assert st == L.LAK_OK
    L.lib().lak_cache_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=7, hkv=2), L.LAK_EINVAL),          # Hq not a multiple of Hkv
    (dict(hq=34, hkv=2), L.LAK_EUNSUPPORTED),   # group of 17 heads
    (dict(d=96), L.LAK_EUNSUPPORTED),
    (dict(page=48), L.LAK_EUNSUPPORTED),
    (dict(num_pages=0), L.LAK_EINVAL),
    (dict(dtype=7), L.LAK_EINVAL),
])
def test_create_rejects(kw, code):
    st, _ = _create(**kw)
    assert st == code
    assert L.lib().lak_last_error().decode()


def test_allocator_reset_grow_and_ragged():
    st, h = _create(num_pages=64, max_batch=4, max_pages=16, page=16)
    assert st == L.LAK_OK
    lib = L.lib()
    lens = (C.c_int32 * 3)(0, 16, 33)
    L.check(lib.lak_seq_reset(h, 3, lens, 0, None), "reset")
    assert _lens(h) == [0, 16, 33]
    assert [len(_pages(h, b)) for b in range(3)] == [0, 1, 3]
    assert lib.lak_free_pages(h) == 60
    # pages are handed out in ascending order and never shared
    allp = _pages(h, 1) + _pages(h, 2)
    assert allp == [0, 1, 2, 3]
    # step: T = 1, 17, 34 -> sequences 0 and 1 open a page, 2 stays in page 2
    L.check(lib.lak_step_begin(h, None), "step")
    assert _lens(h) == [1, 17, 34]
    assert [len(_pages(h, b)) for b in range(3)] == [1, 2, 3]
    assert lib.lak_free_pages(h) == 58
    for _ in range(15):
        L.check(lib.lak_step_begin(h, None), "step")
    assert _lens(h) == [16, 32, 49] and [len(_pages(h, b)) for b in range(3)] == [1, 2, 4]
    # reserve_tokens pre-allocates pages so later steps take none
    L.check(lib.lak_seq_reset(h, 2, (C.c_int32 * 2)(10, 20), 40, None), "reset")
    assert [len(_pages(h, b)) for b in range(2)] == [4, 4]
    for _ in range(30):
        L.check(lib.lak_step_begin(h, None), "step")
    assert lib.lak_free_pages(h) == 56
    lib.lak_cache_destroy(h)


def test_allocator_out_of_pages_and_limits():
    lib = L.lib()
    st, h = _create(num_pages=4, max_batch=2, max_pages=8, page=16)
    assert st == L.LAK_OK
    assert lib.lak_seq_reset(h, 2, (C.c_int32 * 2)(40, 40), 0, None) == L.LAK_ENOPAGE
    assert lib.lak_step_begin(h, None) == L.LAK_ESTATE  # the failed reset left no batch
    L.check(lib.lak_seq_reset(h, 2, (C.c_int32 * 2)(32, 32), 0, None), "reset")
    assert lib.lak_free_pages(h) == 0
    assert lib.lak_step_begin(h, None) == L.LAK_ENOPAGE
    assert _lens(h) == [32, 32]  # unchanged
    assert "free" in lib.lak_last_error().decode()
    # a sequence may not outgrow max_pages_per_seq
    assert lib.lak_seq_reset(h, 1, (C.c_int32 * 1)(8 * 16 + 1), 0, None) == L.LAK_EINVAL
    assert lib.lak_seq_reset(h, 3, (C.c_int32 * 3)(1, 1, 1), 0, None) == L.LAK_EINVAL  # > max_batch
    assert lib.lak_seq_reset(h, 1, (C.c_int32 * 1)(-1), 0, None) == L.LAK_EINVAL
    lib.lak_cache_destroy(h)


def test_attention_calls_on_metadata_only_cache_fail_cleanly():
    lib = L.lib()
    st, h = _create()
    assert lib.lak_attn_full(h, 0, None, None, None, 1.0, None, None, None, 0, None) == L.LAK_ESTATE
    L.check(lib.lak_seq_reset(h, 1, (C.c_int32 * 1)(5), 0, None), "reset")
    dummy = C.c_void_p(256)
    assert lib.lak_attn_full(h, 0, dummy, None, None, 1.0, dummy, None, dummy, 1 << 20, None) == L.LAK_ESTATE
    assert lib.lak_kv_append(h, 0, dummy, dummy, None) == L.LAK_ESTATE
    assert lib.lak_attn_full(None, 0, dummy, None, None, 1.0, dummy, None, dummy, 1 << 20, None) == L.LAK_EINVAL
    assert lib.lak_workspace_bytes(h) > 0
    assert lib.lak_stack_step(h, None, dummy, 1 << 20, None) == L.LAK_ESTATE
    # the no-allocation variant validates like the workspace call (before any device lookup)
    assert lib.lak_attn_sparse_noalloc(h, 0, dummy, None, None, 1.0, dummy, dummy, 4, 0, dummy, None,
                                       None) == L.LAK_ESTATE
    assert lib.lak_attn_sparse_noalloc(None, 0, dummy, None, None, 1.0, dummy, dummy, 4, 0, dummy, None,
                                       None) == L.LAK_EINVAL
    lib.lak_cache_destroy(h)


def test_workspace_covers_logits_and_partials():
    lib = L.lib()
    st, h = _create(max_batch=4, max_pages=16, page=16, hq=8, hkv=2, d=64)
    ws = lib.lak_workspace_bytes(h)
    # delta scratch per (b, kv head, 16-token sub-tile): one block of G x 16 fp16 weights
    # and G float maxima (G = 4: 144 bytes, padded to 160); plus the (max, sum) split
    # partials [Hq][s_cap][2]
    subtiles = 4 * 2 * (16 * 16 // 16)
    assert ws >= subtiles * 4 * (16 * 2 + 4) + 8 * 2 * 4
    assert ws >= subtiles * 160
    lib.lak_cache_destroy(h)


def _golden(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_kv_bytes_match_pages_llama3_figure():
    for layers, kvh, hd, ctx, batch, eb, lower in _golden("pages_kv_size.txt"):
        b = acc.kv_cache_bytes(int(layers), int(kvh), int(hd), int(ctx), int(batch), int(eb))
        assert b > int(lower)
        assert b == 549_755_813_888  # 2 * 32 * 8 * 128 * 32768 * 128 * 2


def test_tier_bytes_and_selected_tokens():
    # budget K + L pages with a partial last page: (K + L - 1) * P + tail tokens
    assert acc.selected_tokens(8192, 16, 96, 32) == 2048
    assert acc.selected_tokens(8193, 16, 96, 32) == 127 * 16 + 1
    assert acc.selected_tokens(100, 16, 96, 32) == 100        # budget covers the context
    full = acc.full_layer_bytes([8192], 28, 4, 128, 2)
    assert full == 8192 * 4 * 128 * 2 * 2 + 2 * 28 * 128 * 2
    sp = acc.sparse_layer_bytes([8192], 28, 4, 128, 2, 16, 96, 32)
    assert sp == 2048 * 4 * 128 * 2 * 2 + 2 * 28 * 128 * 2 + 4 * 128 * 4
    tiers = ["full", "full", "delta"] + ["sparse"] * 3
    assert acc.attended_tokens([4096], tiers, 16, 64, 8) == 3 * 4096 + 3 * 72 * 16


def test_header_is_plain_c():
    """include/lak.h compiles as C99 (no C++ or HIP types in the ABI) and a C caller
    can name every entry point."""
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    calls = "\n".join(f"  (void)&{n};" for n in _declared_symbols())
    src = f'#include "lak.h"\nint main(void) {{\n{calls}\n  return 0;\n}}\n'
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "use_lak.c")
        with open(path, "w") as f:
            f.write(src)
        r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), path], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share; a request for several exits with a message
    (before touching any GPU) instead of reporting a number it did not measure."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
