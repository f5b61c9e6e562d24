"""The fp32 helpers the decode and scan kernels share, checked exhaustively on
the GPU by selective_state_update_amd/math_probe (built with the library by
__graft_entry__.build()): gfx950's bf16 conversion equals round-to-nearest-even
on every fp32 bit pattern, the decay's exp is within 2 ulp of the correctly
rounded exp wherever that is a normal number (results below 2^-126 may come
out as zero: an absolute error under 1.2e-38), and both exp and softplus keep
zeros, infinities and NaN."""
import math
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "selective_state_update_amd", "math_probe")


@pytest.mark.gpu
def test_shared_math_helpers():
    assert os.path.exists(PROBE), "math_probe is not built (run __graft_entry__.build())"
    print("running math_probe", flush=True)
    res = subprocess.run([PROBE], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stderr
    lines = {ln.split()[0]: ln.split()[1:] for ln in res.stdout.splitlines() if ln.strip()}
    assert lines["bf16_mismatches"][0] == "0"
    ranges = [ln.split() for ln in res.stdout.splitlines() if ln.startswith("exp_range")]
    assert len(ranges) == 2
    for r in ranges:
        f = dict(zip(r[3::2], r[4::2]))
        assert int(f["max_ulp_normal"]) <= 2, r
    e = [float(v) for v in lines["exp_specials"]]
    assert e[0] == 1.0 and e[1] == 1.0 and e[2] == math.inf and e[3] == 0.0 and math.isnan(e[4])
    s = [float(v) for v in lines["softplus_specials"]]
    # softplus(0) = ln 2 within the softplus's stated 4 ulp (ulp at 0.69: 2^-24)
    assert abs(s[0] - math.log(2.0)) <= 4 * 2.0**-24 and abs(s[1] - math.log(2.0)) <= 4 * 2.0**-24
    assert s[2] == math.inf and s[3] == 0.0 and math.isnan(s[4])
