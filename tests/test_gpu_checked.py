"""GPU: the checked library (libmoe_routed_checked.so, include/moe_routed_checked.h), whose kernels
test every global memory access against its buffer, runs every shape and flag combination of the
guard-region test, the allocation-free forward, the row steps, the four full-size workloads and
x just under 4 GiB without a single access outside a buffer, matches the oracle on the default flags, and reports violations when its extents are
taken 16 bytes short. The cases run in one child process (tests/checked_run.py), because the
binding chooses its library once per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_checked_library_finds_no_access_outside_a_buffer():
    lib = os.path.join(ROOT, "mixture_experts_routed_plan_amd", "libmoe_routed_checked.so")
    assert os.path.exists(lib), "the checked library is not built"
    env = dict(os.environ, MOE_ROUTED_LIBRARY="checked")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "checked_run.py")], env=env,
                       capture_output=True, text=True, timeout=900)
    print(r.stdout[-6000:])
    print(r.stderr[-6000:])
    assert r.returncode == 0, "checked run failed (exit %d)" % r.returncode
    assert "all cases clean" in (r.stdout + r.stderr)
