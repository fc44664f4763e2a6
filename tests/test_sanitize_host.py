"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
page allocator, argument validation and error paths of the C ABI, exercised on
metadata-only caches by tests/sanitize/abi_host_check.cpp (no device is touched).  The
library is compiled as usual for gfx950 with the sanitizers on its host side only, plus
LAK_DEBUG_CHECKS, which checks the allocator's invariants (every page id inside the
pool, none held twice, none lost) after every allocation."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "layer_aware_kv_amd", "csrc")
SOURCES = ["api.hip", "kv_kernels.hip", "decode_kernels.hip", "select_kernels.hip"]
# sanitizers on the host code only (each -fsanitize= right after -Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
       "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-DLAK_DEBUG_CHECKS", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_paths_under_asan_ubsan():
    out = os.path.join(ROOT, "_build", "asan")
    os.makedirs(out, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        rc, log = _run([HIPCC, "-x", "hip", *COMMON, *SAN, "-c", src, "-o", obj])
        assert rc == 0, log
        return obj

    srcs = [os.path.join(CSRC, f) for f in SOURCES]
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(out, "abi_host_check.o")
    rc, log = _run([HIPCC, *COMMON, *SAN, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"),
                    "-o", drv])
    assert rc == 0, log
    exe = os.path.join(out, "abi_host_check")
    rc, log = _run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, drv, *objs])
    assert rc == 0, log
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, log = _run([exe], env=env, timeout=300)
    assert rc == 0, log
    assert "abi host check ok" in log
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
