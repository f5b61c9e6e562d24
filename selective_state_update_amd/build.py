"""Build libssu.so (HIP, gfx950) in-tree with hipcc.

    python selective_state_update_amd/build.py

The library lands next to this file, where the Python binding loads it.
Flags: gfx950 code only; -O3; no floating-point contraction beyond the
explicit fmaf calls in the kernel (so each result is rounded exactly as the
source states); packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n) for n in ("ssu.hip", "block_copy.hip", "scan.hip")]
LIB = os.path.join(HERE, "libssu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra=(), out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("libssu build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = [ln for ln in res.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln
             and "not a recognized feature" not in ln]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(HERE, "csrc", "valu_rate_probe.hip")
PROBE = os.path.join(HERE, "valu_rate_probe")
MATH_PROBE_SRC = os.path.join(HERE, "csrc", "math_probe.hip")
MATH_PROBE = os.path.join(HERE, "math_probe")


def _build_program(src: str, out: str) -> str:
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [HIPCC, *flags, "-I", os.path.join(HERE, "csrc"), "-o", out + ".tmp", src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("probe build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(out + ".tmp", out)
    return out


def build_probe(out: str = PROBE) -> str:
    """The standalone probe programs, with the library's code-generation flags:
    the VALU issue-rate probe (returned) and the exhaustive check of the
    kernels' shared fp32 helpers (math_probe)."""
    _build_program(MATH_PROBE_SRC, MATH_PROBE)
    return _build_program(PROBE_SRC, out)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe())
