"""Build the CPU oracle (test infrastructure) into oracle/libssu_ref.so with gcc.

Plain C, -O2, no fast-math and no floating-point contraction, so every fp64
operation in ssu_ref.c rounds exactly as written. OpenMP parallelises over the
independent (request, head) units only.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssu_ref.c")
LIB_PATH = os.path.join(HERE, "libssu_ref.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build_oracle(src: str = SRC, out: str = LIB_PATH, extra_flags=(), quiet: bool = False) -> str:
    """Compile ``src`` into the shared library ``out`` and return its path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, src, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if res.stderr and not quiet:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())
