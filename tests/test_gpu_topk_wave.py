"""The one-wave-per-row selector (keys in registers, per-lane LDS histograms, wave
ballots for the ordered write-out) is built beside the workgroup selector but is not
the default: the workgroup selector measured faster at every row length tried.  This
runs the selector parity tests -- the selector fed the oracle's scores (exact, ties
included) and the delta-layer selections against the oracle within the boundary band --
in one child process with LAK_TUNE_TOPK_WAVE_KPL=128, so that every row of up to 8192
candidate pages takes the one-wave selector (tuning knobs are read once per process)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_selection_parity_with_the_one_wave_selector():
    env = dict(os.environ, LAK_TUNE_TOPK_WAVE_KPL="128")
    print("child: test_gpu_kernels.py -k 'page_select or delta_select' with LAK_TUNE_TOPK_WAVE_KPL=128", flush=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_gpu_kernels.py"), "-k", "page_select or delta_select",
                        "--timeout", "300", "--timeout-method", "thread"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=570)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, "one-wave selector: child pytest failed"
    assert " passed" in r.stdout and "failed" not in r.stdout
