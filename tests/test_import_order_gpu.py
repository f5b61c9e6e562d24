"""The package imported before torch: libssu must still share torch's HIP
runtime (a second runtime in the process sees no device)."""
import os
import subprocess
import sys

import pytest

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import selective_state_update_amd as ssu   # first, as a user might
import torch

H, P, N, bs = 2, 64, 128, 3
g = torch.Generator(device="cpu").manual_seed(5)
state = torch.randn(4, H, P, N, generator=g).cuda()
x = torch.randn(bs, H, P, generator=g).bfloat16().cuda()
B = torch.randn(bs, 1, N, generator=g).bfloat16().cuda()
C = torch.randn(bs, 1, N, generator=g).bfloat16().cuda()
dt = torch.randn(bs, H, generator=g).bfloat16().cuda()
A = -torch.rand(H, generator=g).cuda() - 0.5
idx = torch.tensor([2, 0, 3], dtype=torch.int32).cuda()
out = ssu.selective_state_update(state, x, dt, A, B, C, state_batch_indices=idx)
torch.cuda.synchronize()
assert torch.isfinite(out.float()).all()

u = torch.randn(1, 8, 100, generator=g).half().cuda()
delta = torch.randn(1, 8, 100, generator=g).half().cuda()
Bs = torch.randn(1, 1, 16, 100, generator=g).half().cuda()
Cs = torch.randn(1, 1, 16, 100, generator=g).half().cuda()
As = -torch.rand(8, 16, generator=g).cuda() - 0.5
h = torch.zeros(1, 8, 16).cuda()
y = ssu.selective_scan(u, delta, As, Bs, Cs, h)
torch.cuda.synchronize()
assert torch.isfinite(y.float()).all()
print("ok")
"""


def test_package_imported_before_torch():
    gu.require_gpu()
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-1000:] + r.stderr[-3000:]
