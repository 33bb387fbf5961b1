"""The debug build's device bounds checks on every decode path (GPU).

libmlra_debug.so is the same sources built with MLRA_DEBUG_BOUNDS: the
decode and merge kernels check the indices the split-KV plan hands them and
record a failure, which the call then returns as MLRA_ERR_BOUNDS (see
mlra_bounds_checks in include/mlra.h). The binding loads one library per
process, so the cases run in one child process with MLRA_LIB pointing at the
debug build (tests/_debug_bounds_run.py).
"""

import os
import subprocess
import sys

import pytest

import branch_rank_amd as br

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_decode_path_passes_the_device_bounds_checks():
    assert os.path.exists(br.DEBUG_LIB_PATH), "libmlra_debug.so is not built"
    env = dict(os.environ, MLRA_LIB=br.DEBUG_LIB_PATH)
    r = subprocess.run([sys.executable, "-u", "-m", "tests._debug_bounds_run"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    assert r.stdout.strip().endswith("ok")
