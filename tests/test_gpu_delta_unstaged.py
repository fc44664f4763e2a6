"""The delta decode writes its page-score scratch straight to global memory when a
split's blocks do not fit the LDS stage (large splits, e.g. batch 16 past ~87k tokens
at G = 7).  Every other test plans small splits, which are staged, so this runs the
delta-select parity tests again in one child process with staging switched off
(LAK_TUNE_DELTA_LDS=0; tuning knobs are read once per process): MAX and SUM, GROUP
and ALL, every shape of test_gpu_kernels, against the oracle as before."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_delta_select_with_unstaged_scratch():
    env = dict(os.environ, LAK_TUNE_DELTA_LDS="0")
    print("child: test_gpu_kernels.py -k 'delta_select or wide_logit' with LAK_TUNE_DELTA_LDS=0", flush=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_gpu_kernels.py"), "-k", "delta_select or wide_logit",
                        "--timeout", "300", "--timeout-method", "thread"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=570)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, "unstaged delta scratch: child pytest failed"
    assert " passed" in r.stdout and "failed" not in r.stdout
