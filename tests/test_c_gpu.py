"""libssu from plain C on the GPU (tests/c_gpu_check.c): the system ROCm HIP
runtime rather than torch's, a decode step and a two-chunk scan against the
oracle under the same acceptance rules as the Python parity tests."""
import os
import subprocess

import pytest

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_gpu_check")


def test_c_caller_on_gpu_matches_oracle():
    gu.require_gpu()
    assert os.path.exists(EXE), "tests/c_gpu_check is not built (__graft_entry__.build())"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=180)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
