"""Host-side checks of the benchmark's measurement arithmetic."""
import os
import subprocess
import sys

import numpy as np

import bench
import ssu_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p1_b200_kernel_timings.txt")


def _golden():
    rows, tbps = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "tbps":
            tbps = (int(f[1]), float(f[2]), float(f[3]))
        else:
            rows.append((int(f[0]), float(f[1]), float(f[2])))
    return rows, tbps


def test_byte_formula_reproduces_the_pages_bandwidth():
    """The page prints about 3.1 -> 6.3 TB/s at batch 512 for 173.5 -> 85.7 us;
    the state bytes of a call (fp32, read + written) over those times must give
    the same figures to the printed digit, and so must the full algorithmic
    byte count (the small operands add under 0.5%)."""
    rows, (bs, tb_base, tb_pr) = _golden()
    us = {r[0]: (r[1], r[2]) for r in rows}
    base_us, pr_us = us[bs]
    for nbytes in (bench.state_bytes(16, 64, 128, bs), bench.algorithmic_bytes(16, 64, 128, 1, bs)):
        assert round(nbytes / (base_us * 1e-6) / 1e12, 1) == tb_base
        assert round(nbytes / (pr_us * 1e-6) / 1e12, 1) == tb_pr
    assert bench.algorithmic_bytes(16, 64, 128, 1, bs) / bench.state_bytes(16, 64, 128, bs) < 1.005


def test_byte_formula_terms():
    H, P, N, G, bs = 3, 16, 32, 1, 5
    got = bench.algorithmic_bytes(H, P, N, G, bs)
    parts = dict(state=8 * bs * H * P * N, x=2 * bs * H * P, BC=2 * 2 * bs * G * N, dt=2 * bs * H,
                 idx=4 * bs, params=3 * 4 * H, out=2 * bs * H * P)
    assert got == sum(parts.values())


def test_rotation_sets_are_disjoint_and_cold():
    per_call = 512 * 16 * 64 * 128 * 4
    K, sets = si.rotation_sets(per_call, 512, bench.ROTATION_BYTES, seed=3)
    assert K * per_call >= 3 * 256 * 1024 * 1024
    flat = sets.ravel()
    assert len(np.unique(flat)) == flat.size == K * 512
    assert flat.min() == 0 and flat.max() == K * 512 - 1
    K8, _ = si.rotation_sets(8 * 16 * 64 * 128 * 4, 8, bench.ROTATION_BYTES, seed=1)
    assert K8 == 192


def test_sweep_grid_is_920_points():
    pts = si.sweep_points()
    assert len(pts) == 920
    assert {h for h, _ in pts} == {8, 16, 32, 64, 128}
    bss = sorted({b for _, b in pts})
    assert bss[:64] == list(range(1, 65)) and bss[64:] == list(range(72, 1025, 8))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_copy_byte_formula_reproduces_the_pages_tables():
    """The vLLM page prints latency and GB/s for the same runs; 2 x reqs x the
    per-request block bytes (24 x (2 MiB + 80 KiB)) over the latency must give
    its GB/s, so the bench's copy metric is the page's."""
    path = os.path.join(os.path.dirname(__file__), "golden", "p2_copy_kernel.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 6
    for gpu, reqs, us, gbps in rows:
        got = bench.copy_gbps(int(reqs), float(us) * 1e-6)
        assert abs(got - float(gbps)) <= 0.001 * float(gbps), (gpu, reqs, got, gbps)
    assert abs(bench.copy_bytes_per_request() / 2 ** 20 - 49.88) < 0.01


def test_scan_byte_formulas():
    """The scan's algorithmic bytes, written out term by term for the page's
    shape (batch 1, dim 1024, d_state 16, one group, 4096 tokens, 16-bit io),
    and one launch's share at a static chunk of 512 tokens."""
    import bench

    bs, dim, N, G, L = 1, 1024, 16, 1, 4096
    u = delta = out = 2 * bs * dim * L
    Bb = Cb = 2 * bs * G * N * L
    state_rw = 2 * 4 * bs * dim * N
    params = 4 * dim * N + 4 * dim + 4 * dim   # A, D, delta_bias
    assert bench.scan_bytes(bs, dim, N, G, L) == u + delta + out + Bb + Cb + state_rw + params == 25_632_768
    per_launch = 3 * 2 * dim * 512 + 2 * 2 * N * 512 + state_rw + params
    assert bench.scan_launch_bytes(bs, dim, N, G, 512) == per_launch == 3_383_296
    assert bench.scan_elements(bs, dim, N, L) == 67_108_864


def test_shape_list_parsing():
    assert bench.parse_shapes("16x64x128x1x512,8X32x16x2x4") == [(16, 64, 128, 1, 512), (8, 32, 16, 2, 4)]
    for bad in ("16x64x128x1", "16x64x128x1x0", "16x64x128xGx512"):
        try:
            bench.parse_shapes(bad)
        except (SystemExit, ValueError):
            continue
        raise AssertionError(f"accepted {bad!r}")
