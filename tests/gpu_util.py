"""Helpers for the GPU tests: move a seeded Problem to the device, run libssu
through its C ABI, and compare with the CPU oracle under the acceptance rules
of tests/tolerance.py."""
from __future__ import annotations

import numpy as np

import ssu_inputs as si

from . import tolerance as tol


def torch_mod():
    import torch

    return torch


def require_gpu():
    import pytest

    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    # the product path must be the HIP library; importing it fails loudly if unbuilt
    import selective_state_update_amd  # noqa: F401


def bf16_tensor(a: np.ndarray, device):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def bits(t) -> np.ndarray:
    """bf16 tensor -> uint16 numpy bit patterns."""
    torch = torch_mod()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceProblem:
    """Device copies of a Problem's operands, laid out as the kernel workload
    describes them: x/B/C as views into one packed bf16 tensor, per-head
    parameters as [H] tensors (broadcast with stride 0 by the binding)."""

    def __init__(self, p: si.Problem, device="cuda", pool=None):
        torch = torch_mod()
        H, P, N, G, bs = p.nheads, p.headdim, p.dstate, p.ngroups, p.batch
        self.p = p
        self.device = device
        self.pool = pool if pool is not None else torch.from_numpy(p.pool).to(device)
        self.xbc = bf16_tensor(p.xbc, device)
        row = self.xbc.stride(0)
        self.x = self.xbc.as_strided((bs, H, P), (row, P, 1), 0)
        self.B = self.xbc.as_strided((bs, G, N), (row, N, 1), H * P)
        self.C = self.xbc.as_strided((bs, G, N), (row, N, 1), H * P + G * N)
        self.dt = bf16_tensor(p.dt, device)
        self.A = torch.from_numpy(p.A).to(device)
        self.D = torch.from_numpy(p.D).to(device)
        self.dt_bias = torch.from_numpy(p.dt_bias).to(device)
        self.idx = torch.from_numpy(p.idx).to(device)
        self.out = torch.empty((bs, H, P), dtype=torch.bfloat16, device=device)

    def handle(self, tile=-1):
        import selective_state_update_amd as ssu

        p = self.p
        return ssu.Handle(p.nheads, p.headdim, p.dstate, p.ngroups, p.dt_softplus, tile)

    def run(self, handle=None, tile=-1, use_bias=True, use_D=True, idx=None, out=None):
        h = handle or self.handle(tile)
        out = self.out if out is None else out
        h.update(self.pool, self.idx if idx is None else idx, self.x, self.B, self.C, self.dt, self.A,
                 self.D if use_D else None, self.dt_bias if use_bias else None, out)
        return out


def oracle_step(ref, p: si.Problem, pool_np: np.ndarray, use_bias=True, use_D=True, idx=None):
    """Run the oracle on a host copy of the pool (updated in place)."""
    return ref.run(pool_np, p.idx if idx is None else idx, p.x, p.B, p.C, p.dt, p.A,
                   p.dt_bias if use_bias else None, p.D if use_D else None, p.dt_softplus)


def assert_state(gpu_state: np.ndarray, ref_state: np.ndarray, what=""):
    bad = tol.state_violations(gpu_state, ref_state)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} state elements out of tolerance; first at {i}: "
                             f"gpu={gpu_state[i]!r} ref={ref_state[i]!r}")


def assert_out(out_bits: np.ndarray, r: dict, what=""):
    fail, floor_passes = tol.out_check(out_bits, r["out"], r["y"], r["tau"])
    if fail.any():
        i = tuple(np.argwhere(fail)[0])
        raise AssertionError(f"{what}: {int(fail.sum())} outputs out of tolerance; first at {i}: "
                             f"gpu={tol.bf16_to_f64(out_bits[i])!r} ref_bits={r['out'][i]:#06x} "
                             f"y={r['y'][i]!r} tau={r['tau'][i]!r}")
    return floor_passes


def compare_full(ref, dp: DeviceProblem, pool_before: np.ndarray, out_t, what="", **kw):
    """Oracle on the whole problem; GPU pool and out checked element by element,
    untouched slots bitwise."""
    p = dp.p
    pool_ref = pool_before.copy()
    r = oracle_step(ref, p, pool_ref, **kw)
    pool_gpu = dp.pool.cpu().numpy()
    idx = p.idx if kw.get("idx") is None else kw["idx"]
    live = idx[(idx >= 0) & (idx < p.pool_slots)]
    rows = np.nonzero((idx >= 0) & (idx < p.pool_slots))[0]
    assert_state(pool_gpu[live], r["state"][rows], what)
    untouched = np.setdiff1d(np.arange(p.pool_slots), live)
    assert np.array_equal(pool_gpu[untouched].view(np.uint32), pool_before[untouched].view(np.uint32)), \
        f"{what}: untouched slots changed"
    out_bits = bits(out_t)
    floor = assert_out(out_bits[rows], {k: r[k][rows] for k in ("out", "y", "tau")}, what)
    return r, pool_gpu, out_bits, floor
