"""The split-K decode kernel loads U sub-tiles per batch (U = 1, 2 or 4, a template
parameter).  The default plans, for bf16 pools, U = 1 on the full and delta tiers and,
on the sparse tier, U = 2 only when a wave's whole share is at most two sub-tiles; for
fp8 pools U = 2 on the sparse tier and on a delta launch whose LDS stage limits
occupancy.  So that every batch depth is checked
against the oracle on every tier and pool type, this runs the parity tests again in
child processes with the depth forced (tuning knobs are read once per process): bf16
attention tests of test_gpu_kernels with U = 2 on the full and delta tiers and U = 1 on
the sparse tier, and with U = 4 on the sparse tier; the fp8 tests of test_gpu_fp8 with
U = 1 on every tier, and with U = 2 on the delta tier (the default takes it only where
the LDS stage limits occupancy: the full-size stack tests) -- fp32 pools always take
U = 1 -- against the oracle exactly as the default run is."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SELECT = "full_attention or delta_select or sparse or fused or wide_logit or edge_cases or invalid_selection"


def _run_child(env_over, test_file="test_gpu_kernels.py", select=SELECT):
    env = dict(os.environ, **env_over)
    print(f"child: {test_file} -k '{select}' with {env_over}", flush=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file), "-k", select,
                        "--timeout", "300", "--timeout-method", "thread"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=570)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, f"{env_over}: child pytest failed"
    assert " passed" in r.stdout and "failed" not in r.stdout


@pytest.mark.timeout(600)
def test_two_subtiles_per_batch_full_delta_one_sparse():
    _run_child({"LAK_TUNE_DECODE_BATCH": "2", "LAK_TUNE_DELTA_BATCH": "2", "LAK_TUNE_SPARSE_BATCH": "1"})


@pytest.mark.timeout(600)
def test_four_subtiles_per_batch_sparse():
    _run_child({"LAK_TUNE_SPARSE_BATCH": "4"})


@pytest.mark.timeout(600)
def test_one_subtile_per_batch_fp8():
    _run_child({"LAK_TUNE_DECODE_BATCH": "1", "LAK_TUNE_DELTA_BATCH": "1", "LAK_TUNE_SPARSE_BATCH": "1"},
               "test_gpu_fp8.py", "fp8")


@pytest.mark.timeout(600)
def test_two_subtiles_per_batch_fp8_delta():
    _run_child({"LAK_TUNE_DELTA_BATCH": "2"}, "test_gpu_fp8.py", "fp8")
