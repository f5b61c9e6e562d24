"""include/ssu.h from C: compiled as C11 with gcc, linked against the built
libssu.so and run on inputs that need no GPU (tests/c_abi_check.c)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "selective_state_update_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_header_compiles_as_c_and_every_entry_point_links(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libssu.so")):
        pytest.fail("libssu.so is not built")
    exe = tmp_path / "c_abi_check"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe),
           "-L", LIBDIR, "-Wl,-rpath," + LIBDIR, "-l:libssu.so"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
