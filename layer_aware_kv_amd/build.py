"""Builds the gfx950 shared libraries in-tree with hipcc.

    python -m layer_aware_kv_amd.build      # liblak.so and workload/libworkload.so

Every source is compiled each time (the build is the "does it build" check).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for all device code.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

LIBS = {
    "lak": dict(
        srcs=[os.path.join(PKG, "csrc", f) for f in
              ("api.hip", "kv_kernels.hip", "decode_kernels.hip", "select_kernels.hip")],
        includes=[os.path.join(ROOT, "include"), os.path.join(PKG, "csrc")],
        # no FMA contraction: every tier rounds the same products the same way
        extra=["-ffp-contract=off"],
        out=os.path.join(PKG, "liblak.so")),
    "workload": dict(
        srcs=[os.path.join(ROOT, "workload", "csrc", "fill.hip")],
        includes=[],
        extra=["-ffp-contract=off"],
        out=os.path.join(ROOT, "workload", "libworkload.so")),
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), "\n".join(lines)))
    return "\n".join(lines)


def build_lib(name: str, verbose: bool = False) -> str:
    spec = LIBS[name]
    bdir = os.path.join(ROOT, "_build", name)
    os.makedirs(bdir, exist_ok=True)
    incs = sum((["-I", i] for i in spec["includes"]), [])

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        out = _run([HIPCC, *COMMON, *spec["extra"], *incs, "-c", src, "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(spec["srcs"]))) as ex:
        objs = list(ex.map(compile_one, spec["srcs"]))
    tmp = spec["out"] + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    shutil.move(tmp, spec["out"])
    return spec["out"]


def build_all(verbose: bool = False):
    return [build_lib(n, verbose) for n in LIBS]


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
