#!/usr/bin/env python3
"""Benchmark of libssu's decode-step selective_state_update on one MI355X.

Method: the measurement set-up of sglang PR #41223, "[Perf] Mamba2
selective_state_update up to 2x faster on B200 via 8x1 launch config for
dstate 128", section "Kernel measurement". One graph holds many calls;
consecutive calls work on disjoint sets of state slots, and all the sets
together exceed the last-level cache three times over, so no call finds its
state in cache. (A decoding model's layer meets its state cold in the same
way: once per generated token.) Here the graph is a HIP graph and the
last-level cache is MI355X's 256 MB Infinity Cache: the sets total >= 768 MiB.

A "step" is one ssu_update call over one batch. The default workload is the
headline one: H=16, P=64, N=128, batch 512, fp32 state, bf16 x/B/C as strided
views of one tensor, per-head dt/A/D/dt_bias broadcasts.

Output: one JSON line (see the keys below). `value` is HBM GB/s computed from
the algorithmic bytes of a call; the roofline object prices the kernel against
the 8 TB/s HBM3E peak; cpu_baseline times the fp64 CPU oracle on the host on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config 1|2|3] [--tile T]
    python bench.py --sweep [--heads 16] [--out FILE]   per-point GB/s (no JSON line)
    python bench.py --counters                          short eager run for rocprofv3 --pmc
    python bench.py --summarize-counters DIR --write-profile NAME
    python bench.py --scan 1,2,3 [--chunks 64,...,4096]  selective scan (prefill) per sequence
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import ssu_inputs as si  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
LLC_BYTES = 256 * 1024 * 1024  # MI355X Infinity Cache
ROTATION_BYTES = 3 * LLC_BYTES  # >= 3x the last-level cache
KERNEL_SRCS = [os.path.join(ROOT, "selective_state_update_amd", "csrc", "ssu.hip"),
               os.path.join(ROOT, "selective_state_update_amd", "csrc", "internal.h")]
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "ssu_decode_h16_bs512_counters.md")

WORKLOADS = {
    1: dict(H=16, P=64, N=128, G=1, batch=8),
    2: dict(H=16, P=64, N=128, G=1, batch=128),
    3: dict(H=16, P=64, N=128, G=1, batch=512),
}


def state_bytes(H, P, N, batch):
    """fp32 state read + written once per call."""
    return 8 * batch * H * P * N


def algorithmic_bytes(H, P, N, G, batch):
    """Bytes one call must move: state read+write (fp32), x (bf16), B and C
    (bf16, once per request and group), dt (bf16 per request and head), idx
    (int32), A, D, dt_bias (fp32 per head) and out (bf16)."""
    return (8 * batch * H * P * N + 2 * batch * H * P + 4 * batch * G * N + 2 * batch * H
            + 4 * batch + 12 * H + 2 * batch * H * P)


def scan_source_digest() -> str:
    """Hash of the scan kernel's source (comments and whitespace stripped)."""
    return _digest([os.path.join(ROOT, "selective_state_update_amd", "csrc", "scan.hip"),
                    os.path.join(ROOT, "selective_state_update_amd", "csrc", "internal.h")])


def _digest(files) -> str:
    """Hash of source files with comments and whitespace removed, so that only
    a change to the code itself invalidates counter data."""
    import re

    text = "\n".join(open(f).read() for f in files)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def source_digest() -> str:
    """Hash of the decode kernel's source code (its file and the shared header)."""
    return _digest(KERNEL_SRCS)


# --------------------------------------------------------------------------- #
class Rotation:
    """K disjoint slot sets of `batch` requests over a pool of K*batch slots,
    with per-set x/B/C, dt and out buffers, all resident in HBM."""

    def __init__(self, H, P, N, G, batch, seed, device="cuda", min_bytes=ROTATION_BYTES):
        import torch

        self.H, self.P, self.N, self.G, self.batch = H, P, N, G, batch
        per_call = batch * H * P * N * 4
        self.K, sets = si.rotation_sets(per_call, batch, min_bytes, seed)
        self.pool = torch.empty((self.K * batch, H, P, N), dtype=torch.float32, device=device)
        si.draw_pool_on_device(self.pool, seed)
        self.sets = []
        for k in range(self.K):
            p = si.make_problem(H, P, N, G, batch, self.K * batch, seed * 1000 + k, host_pool=False,
                                idx=sets[k])
            xbc = torch.from_numpy(p.xbc.view(np.int16)).view(torch.bfloat16).to(device)
            row = xbc.stride(0)
            self.sets.append(dict(
                problem=p,
                idx=torch.from_numpy(p.idx).to(device),
                x=xbc.as_strided((batch, H, P), (row, P, 1), 0),
                B=xbc.as_strided((batch, G, N), (row, N, 1), H * P),
                C=xbc.as_strided((batch, G, N), (row, N, 1), H * P + G * N),
                xbc=xbc,
                dt=torch.from_numpy(p.dt.view(np.int16)).view(torch.bfloat16).to(device),
                out=torch.empty((batch, H, P), dtype=torch.bfloat16, device=device),
            ))
        p0 = self.sets[0]["problem"]
        self.A = torch.from_numpy(p0.A).to(device)
        self.D = torch.from_numpy(p0.D).to(device)
        self.dt_bias = torch.from_numpy(p0.dt_bias).to(device)

    def args(self, handle):
        """Prepared ssu_args per set (marshalled once, outside the timed region)."""
        out = []
        for s in self.sets:
            out.append(handle.make_args(self.pool, s["idx"], s["x"], s["B"], s["C"], s["dt"], self.A,
                                        self.D, self.dt_bias, s["out"]))
        return out


def capture(handle, args, first, count):
    """A HIP graph of `count` calls; call i uses set (first + i) mod K."""
    import torch

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        handle.launch(args[first % len(args)])  # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(count):
            handle.launch(args[(first + i) % len(args)])
    return g


def time_graph(g, replays):
    """Seconds for `replays` back-to-back replays, bracketed by events on the
    stream the kernels run on (torch's current stream)."""
    import torch

    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def cpu_oracle_baseline(H, P, N, G, batch, seed, budget_s=20.0):
    """The CPU oracle (fp64, OpenMP over (request, head)) on host cores, on a
    bounded sample: whole calls of the same workload, repeated until about
    `budget_s` seconds have passed (at least 2 calls)."""
    import oracle

    ref = oracle.get()
    threads = len(os.sched_getaffinity(0))
    env_threads = os.environ.get("OMP_NUM_THREADS")
    if env_threads and env_threads.isdigit():
        threads = min(threads, int(env_threads))
    slots = batch  # exactly the slots one call touches
    p = si.make_problem(H, P, N, G, batch, slots, seed)
    times = []
    t_start = time.perf_counter()
    while len(times) < 2 or time.perf_counter() - t_start < budget_s:
        pool = p.pool.copy()
        t0 = time.perf_counter()
        ref.run(pool, p.idx, p.x, p.B, p.C, p.dt, p.A, p.dt_bias, p.D, True, want_state=False,
                want_y=False, nthreads=threads)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    gbs = algorithmic_bytes(H, P, N, G, batch) / med / 1e9
    # the same calls on one core
    one = []
    for _ in range(2):
        pool = p.pool.copy()
        t0 = time.perf_counter()
        ref.run(pool, p.idx, p.x, p.B, p.C, p.dt, p.A, p.dt_bias, p.D, True, want_state=False,
                want_y=False, nthreads=1)
        one.append(time.perf_counter() - t0)
    one_med = statistics.median(one)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} whole calls of H{H} P{P} N{N} batch {batch} (median "
                      f"{med * 1e3:.1f} ms/call, fp64 C oracle, OpenMP {threads} threads, {cpu_model})",
            "us_per_call": round(med * 1e6, 1),
            "one_core": {"value": round(algorithmic_bytes(H, P, N, G, batch) / one_med / 1e9, 3), "unit": "GB/s",
                         "us_per_call": round(one_med * 1e6, 1), "sample": "2 whole calls, 1 thread"}}


def counter_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    if not os.path.exists(COUNTER_PROFILE):
        return None
    fields = {}
    for line in open(COUNTER_PROFILE):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_code_digest") != source_digest():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------- #
def run_bench(a):
    import torch

    import selective_state_update_amd as ssu

    w = WORKLOADS[a.config]
    H, P, N, G, bs = w["H"], w["P"], w["N"], w["G"], w["batch"]
    nbytes = algorithmic_bytes(H, P, N, G, bs)
    torch.cuda.init()
    rot = Rotation(H, P, N, G, bs, seed=a.config)
    h = ssu.Handle(H, P, N, G, True, a.tile)
    tile = h.selected_tile(bs)
    tdesc = ssu.tiles()[tile]
    args = rot.args(h)
    calls = max(20, rot.K)
    g = capture(h, args, 0, calls)
    K_steps = a.steps
    full, tail = divmod(K_steps, calls)
    g_tail = capture(h, args, 0, tail) if tail else None
    torch.cuda.synchronize()
    print(f"# workload H{H} P{P} N{N} G{G} bs{bs}: {nbytes} B/call, K={rot.K} sets, "
          f"{calls} calls/graph, tile {tdesc['name']}", file=sys.stderr, flush=True)

    # The pages' statistic first: median of 5 x (20 replays of the graph).
    # It also carries the chip through the first few hundred dispatches after
    # idle, which run up to ~10% slower than the settled rate (clock and power
    # state), so the timed region below measures the kernel, not that ramp.
    reps = [time_graph(g, 20) / (20 * calls) for _ in range(5)]
    med = statistics.median(reps)

    # warmup: at least W calls
    for _ in range(max(1, -(-a.warmup // calls))):
        g.replay()
    torch.cuda.synchronize()

    # timed region: exactly K steps
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(full):
        g.replay()
    if g_tail is not None:
        g_tail.replay()
    e1.record(st)
    e1.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed = e0.elapsed_time(e1) * 1e-3
    per_call = elapsed / K_steps
    gbs = nbytes / per_call / 1e9

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_oracle_baseline(H, P, N, G, bs, seed=a.config, budget_s=a.cpu_budget)

    traffic = counter_traffic()
    line = {
        "metric": "selective_state_update HBM GB/s (% of peak) + µs/call, H16 P64 N128 bs512",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": a.warmup,
        "ms_per_step": round(per_call * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"selective_state_update decode step H{H} P{P} N{N} G{G} batch {bs}, fp32 state, "
                        f"bf16 x/B/C packed, per-head dt/A/D/dt_bias, {rot.K} disjoint slot sets "
                        f"({rot.K * bs * H * P * N * 4 >> 20} MiB) rotated in a HIP graph of {calls} calls",
            "heads": H, "headdim": P, "dstate": N, "ngroups": G, "batch": bs,
            "tile": tdesc["name"],
        },
        "us_per_call": round(per_call * 1e6, 3),
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "median5_us_per_call": round(med * 1e6, 3),
        "bytes_per_call": nbytes,
        "wall_s": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_sweep(a):
    """GB/s and us/call per (heads, batch) point of the bitwise-sweep grid,
    same rotation method; one text line per point."""
    import torch

    import selective_state_update_amd as ssu

    heads = [int(x) for x in a.heads.split(",")] if a.heads else [8, 16, 32, 64, 128]
    batches = sorted({bs for (_, bs) in si.sweep_points()}) if not a.batches else \
        [int(x) for x in a.batches.split(",")]
    out = open(a.out, "w") if a.out else sys.stdout
    print("heads batch tile K calls us_per_call GBps pct_peak", file=out, flush=True)
    for H in heads:
        for bs in batches:
            rot = Rotation(H, 64, 128, 1, bs, seed=si.sweep_seed(H, bs))
            h = ssu.Handle(H, 64, 128, 1, True, a.tile)
            args = rot.args(h)
            calls = max(20, rot.K)
            g = capture(h, args, 0, calls)
            g.replay()
            torch.cuda.synchronize()
            reps = [time_graph(g, 5) / (5 * calls) for _ in range(3)]
            us = statistics.median(reps) * 1e6
            gbs = algorithmic_bytes(H, 64, 128, 1, bs) / (us * 1e-6) / 1e9
            print(f"{H} {bs} {ssu.tiles()[h.selected_tile(bs)]['name']} {rot.K} {calls} {us:.3f} "
                  f"{gbs:.1f} {100 * gbs / HBM_PEAK_GBS:.2f}", file=out, flush=True)
            del g, rot, args
            torch.cuda.empty_cache()


def run_tile_sweep(a):
    """µs/call and GB/s of every compiled launch configuration for this N and
    P on the chosen workload (same rotation and graph method), one line each."""
    import torch

    import selective_state_update_amd as ssu

    w = WORKLOADS[a.config]
    H, P, N, G, bs = w["H"], w["P"], w["N"], w["G"], w["batch"]
    nbytes = algorithmic_bytes(H, P, N, G, bs)
    rot = Rotation(H, P, N, G, bs, seed=a.config)
    auto = ssu.Handle(H, P, N, G, True, -1).selected_tile(bs)
    out = open(a.out, "w") if a.out else sys.stdout
    prop = torch.cuda.get_device_properties(0)
    info = {k: getattr(prop, k) for k in ("name", "multi_processor_count", "shared_memory_per_multiprocessor",
                                          "shared_memory_per_block", "max_threads_per_multi_processor",
                                          "L2_cache_size") if hasattr(prop, k)}
    print(f"# device {info}", file=out)
    print(f"# H{H} P{P} N{N} bs{bs}: {nbytes} B/call; auto tile {ssu.tiles()[auto]['name']}", file=out)
    print("tile name rows_per_group waves us_per_call GBps pct_peak", file=out, flush=True)
    for t in ssu.tiles():
        if t["dstate"] != N or not ssu.tile_fits(t, H, P):
            continue
        h = ssu.Handle(H, P, N, G, True, t["id"])
        args = rot.args(h)
        calls = max(20, rot.K)
        g = capture(h, args, 0, calls)
        g.replay()
        torch.cuda.synchronize()
        reps = [time_graph(g, 10) / (10 * calls) for _ in range(5)]
        us = statistics.median(reps) * 1e6
        gbs = nbytes / (us * 1e-6) / 1e9
        print(f"{t['id']} {t['name']} {t['rows_per_group']} {t['waves']} {us:.3f} {gbs:.1f} "
              f"{100 * gbs / HBM_PEAK_GBS:.2f}", file=out, flush=True)
        del g


def parse_shapes(spec):
    """'HxPxNxGxB,...' -> [(H, P, N, G, batch), ...]."""
    shapes = []
    for item in spec.split(","):
        f = [int(v) for v in item.lower().split("x")]
        if len(f) != 5 or min(f) < 1:
            raise SystemExit(f"--shapes: '{item}' is not HxPxNxGxBATCH")
        shapes.append(tuple(f))
    return shapes


def run_shapes(a):
    """The decode step at other shapes (d_state, headdim, groups, heads,
    batch), same rotation and graph method as the headline: one line per
    shape with the library's launch configuration, and with --tile-sweep one
    line per compiled configuration of that d_state."""
    import torch

    import selective_state_update_amd as ssu

    out = open(a.out, "w") if a.out else sys.stdout
    print("H P N G batch state_MiB tile us_per_call GBps pct_peak", file=out, flush=True)
    for (H, P, N, G, bs) in parse_shapes(a.shapes):
        nbytes = algorithmic_bytes(H, P, N, G, bs)
        rot = Rotation(H, P, N, G, bs, seed=7000 + H + P + N + G + bs)
        auto = ssu.Handle(H, P, N, G, True, -1).selected_tile(bs)
        ids = [auto]
        if a.tile_sweep:
            ids += [t["id"] for t in ssu.tiles()
                    if t["dstate"] == N and ssu.tile_fits(t, H, P) and t["id"] != auto]
        for tid in ids:
            h = ssu.Handle(H, P, N, G, True, tid)
            args = rot.args(h)
            calls = max(20, rot.K)
            g = capture(h, args, 0, calls)
            g.replay()
            torch.cuda.synchronize()
            reps = [time_graph(g, 10) / (10 * calls) for _ in range(5)]
            us = statistics.median(reps) * 1e6
            gbs = nbytes / (us * 1e-6) / 1e9
            name = ssu.tiles()[tid]["name"] + ("*" if tid == auto else "")  # * = the library's choice
            print(f"{H} {P} {N} {G} {bs} {state_bytes(H, P, N, bs) / 2 ** 21:.0f} {name} {us:.3f} {gbs:.1f} "
                  f"{100 * gbs / HBM_PEAK_GBS:.2f}", file=out, flush=True)
            del g, args
        del rot
        torch.cuda.empty_cache()
        if not a.no_cpu_baseline:
            cb = cpu_oracle_baseline(H, P, N, G, bs, seed=7000 + H + P + N + G + bs, budget_s=2.0)
            print(f"# cpu oracle (fp64, {cb['cores']} threads): {cb['us_per_call'] / 1e3:.2f} ms per call, "
                  f"{cb['value']:.1f} GB/s", file=out, flush=True)


def run_copy_ceiling(a):
    """Attainable read+write HBM bandwidth on this machine: plain device copies of
    the headline call's state volume (256 MiB read + 256 MiB written), rotated
    over buffers totalling >= 3x the last-level cache, timed like the decode
    kernel (HIP graph of 20 calls, median of 5 x 20 replays)."""
    import torch

    nelem = 64 * 1024 * 1024  # 256 MiB of fp32
    nbuf = 4
    src = [torch.empty(nelem, device="cuda").normal_() for _ in range(nbuf)]
    dst = [torch.empty(nelem, device="cuda") for _ in range(nbuf)]
    ops = {
        "copy_(hipMemcpy)": lambda i: dst[i].copy_(src[i]),
        "mul(elementwise)": lambda i: torch.mul(src[i], 2.0, out=dst[i]),
        "read-only(sum)": lambda i: src[i].sum(),
    }
    for name, op in ops.items():
        for i in range(nbuf):
            op(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        try:
            with torch.cuda.graph(g):
                for i in range(20):
                    op(i % nbuf)
        except Exception as e:  # noqa: BLE001 - report and go on
            print(f"{name}: capture failed: {e}", flush=True)
            continue
        g.replay()
        torch.cuda.synchronize()
        reps = [time_graph(g, 20) / (20 * 20) for _ in range(5)]
        us = statistics.median(reps) * 1e6
        moved = nelem * 4 * (1 if name.startswith("read-only") else 2)
        print(f"ceiling {name}: {us:.2f} us per {moved >> 20} MiB moved -> {moved / us / 1e3:.1f} GB/s "
              f"({100 * moved / us / 1e3 / HBM_PEAK_GBS:.1f}% of 8 TB/s)", flush=True)


def time_graph_on(g, replays, stream):
    """Seconds for `replays` replays of a graph captured on `stream`, with
    events recorded on that stream."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def tokens_bytes(H, P, N, G, batch, K):
    """Bytes of one K-token call: the state read and written once, then K
    tokens' x, B, C, dt and out, plus idx and the per-head parameters."""
    per_token = 2 * batch * H * P + 4 * batch * G * N + 2 * batch * H + 2 * batch * H * P
    return 8 * batch * H * P * N + K * per_token + 4 * batch + 12 * H


def run_tokens(a):
    """K decode tokens per request in one launch (ssu_update_tokens) at the
    chosen workload, same rotation method; one line per K."""
    import torch

    import selective_state_update_amd as ssu

    w = WORKLOADS[a.config]
    H, P, N, G, bs = w["H"], w["P"], w["N"], w["G"], w["batch"]
    out = open(a.out, "w") if a.out else sys.stdout
    print("tokens us_per_call us_per_token GBps pct_peak tokens_per_s", file=out, flush=True)
    for K in [int(k) for k in a.tokens.split(",")]:
        rot = Rotation(H, P, N, G, bs, seed=a.config)
        h = ssu.Handle(H, P, N, G, True, a.tile)
        args = []
        for s in rot.sets:
            p = s["problem"]
            rng = np.random.Generator(np.random.PCG64([a.config, K]))
            xbc = torch.from_numpy(si.bf16_bits(rng.standard_normal((bs, K, p.xbc.shape[1]), dtype=np.float32))
                                   .view(np.int16)).view(torch.bfloat16).cuda()
            row = xbc.shape[2]
            dt = torch.from_numpy(si.bf16_bits(rng.standard_normal((bs, K, H), dtype=np.float32))
                                  .view(np.int16)).view(torch.bfloat16).cuda()
            o = torch.empty((bs, K, H, P), dtype=torch.bfloat16, device="cuda")
            s["tok"] = (xbc, dt, o)
            args.append(h.make_tokens_args(
                rot.pool, s["idx"], xbc.as_strided((bs, K, H, P), (K * row, row, P, 1), 0),
                xbc.as_strided((bs, K, G, N), (K * row, row, N, 1), H * P),
                xbc.as_strided((bs, K, G, N), (K * row, row, N, 1), H * P + G * N), dt, rot.A, rot.D,
                rot.dt_bias, o))
        calls = max(20, rot.K)
        g = capture(h, args, 0, calls)
        g.replay()
        torch.cuda.synchronize()
        us = statistics.median([time_graph(g, 10) / (10 * calls) for _ in range(5)]) * 1e6
        nb = tokens_bytes(H, P, N, G, bs, K)
        gbs = nb / (us * 1e-6) / 1e9
        print(f"{K} {us:.3f} {us / K:.3f} {gbs:.1f} {100 * gbs / HBM_PEAK_GBS:.2f} {bs * K / (us * 1e-6):.4g}",
              file=out, flush=True)
        del g, rot, args
        torch.cuda.empty_cache()
        if not a.no_cpu_baseline:
            # the CPU oracle on one K-token call of this workload, for context
            import oracle

            base = si.make_problem(H, P, N, G, bs, bs, a.config)
            rng = np.random.Generator(np.random.PCG64([a.config, K]))
            xs = si.bf16_bits(rng.standard_normal((K, bs, H, P), dtype=np.float32))
            bcs = si.bf16_bits(rng.standard_normal((K, bs, G, N), dtype=np.float32))
            dts = si.bf16_bits(rng.standard_normal((K, bs, H), dtype=np.float32))
            threads = len(os.sched_getaffinity(0))
            pool = base.pool.copy()
            t0 = time.perf_counter()
            oracle.get().run(pool, base.idx, xs, bcs, bcs, dts, base.A, base.dt_bias, base.D, True,
                             want_state=False, want_y=False, nthreads=threads)
            print(f"# cpu oracle (fp64, {threads} threads): {(time.perf_counter() - t0) * 1e3:.1f} ms for one "
                  f"{K}-token call", file=out, flush=True)


# Per-request state blocks of the copy workload (vLLM state-block copy page,
# "Test Plan"): 24 layers x (temporal fp32 2 MiB + conv bf16 80 KiB).
COPY_LAYERS = 24
COPY_TEMPORAL_BYTES = 2 * 1024 * 1024
COPY_CONV_BYTES = 80 * 1024


def copy_bytes_per_request():
    return COPY_LAYERS * (COPY_TEMPORAL_BYTES + COPY_CONV_BYTES)


def copy_gbps(nreqs, seconds):
    """Read + written bytes per second, in GB/s (the page's convention)."""
    return 2 * nreqs * copy_bytes_per_request() / seconds / 1e9


def run_copy_blocks(a):
    """ssu_copy_blocks on the page's layout, reqs from --copy-blocks; disjoint
    block sets >= 768 MiB rotated in a HIP graph (cold HBM), median of 5 x 10
    replays. One line per request count."""
    import torch

    import selective_state_update_amd as ssu

    out = open(a.out, "w") if a.out else sys.stdout
    print("reqs K calls us_per_call GBps pct_peak tile", file=out, flush=True)
    per_req = copy_bytes_per_request()
    for nreqs in [int(r) for r in a.copy_blocks.split(",")]:
        K = max(1, -(-ROTATION_BYTES // (nreqs * per_req)))
        nblocks = 2 * K * nreqs
        g = torch.Generator(device="cuda")
        g.manual_seed(nreqs)
        temporal = [torch.empty((nblocks, COPY_TEMPORAL_BYTES // 4), device="cuda").normal_(generator=g)
                    for _ in range(COPY_LAYERS)]
        conv = [torch.empty((nblocks, COPY_CONV_BYTES // 2), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
                for _ in range(COPY_LAYERS)]
        tensors = temporal + conv
        descs = ssu.block_tensors(tensors)
        rng = np.random.Generator(np.random.PCG64([nreqs, 7]))
        perm = rng.permutation(nblocks).astype(np.int32).reshape(K, 2, nreqs)
        ids = [(torch.from_numpy(perm[k, 0].copy()).cuda(), torch.from_numpy(perm[k, 1].copy()).cuda())
               for k in range(K)]
        calls = max(20, K)
        ssu.copy_blocks(tensors, *ids[0], tile=a.tile, descs=descs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(calls):
                ssu.copy_blocks(tensors, *ids[i % K], tile=a.tile, descs=descs)
        graph.replay()
        torch.cuda.synchronize()
        us = statistics.median([time_graph(graph, 10) / (10 * calls) for _ in range(5)]) * 1e6
        gbs = copy_gbps(nreqs, us * 1e-6)
        name = ssu.copy_tiles()[a.tile] if a.tile >= 0 else "default"
        print(f"{nreqs} {K} {calls} {us:.2f} {gbs:.1f} {100 * gbs / HBM_PEAK_GBS:.2f} {name}", file=out, flush=True)
        del graph, tensors, temporal, conv, ids
        torch.cuda.empty_cache()
        if not a.no_cpu_baseline:
            # the CPU oracle (a memcpy loop) on one call of the same layout, for context
            import oracle

            host = [np.zeros((2 * nreqs, COPY_TEMPORAL_BYTES // 4), dtype=np.float32) for _ in range(COPY_LAYERS)] + \
                   [np.zeros((2 * nreqs, COPY_CONV_BYTES // 2), dtype=np.uint16) for _ in range(COPY_LAYERS)]
            for t in host:
                t.fill(1)  # touch the pages before timing
            src = np.arange(nreqs, dtype=np.int32)
            dst = src + nreqs
            t0 = time.perf_counter()
            oracle.get().copy_blocks(host, src, dst)
            sec = time.perf_counter() - t0
            print(f"# cpu oracle (memcpy loop, 1 thread): {sec * 1e3:.1f} ms for one call of {nreqs} requests "
                  f"({copy_gbps(nreqs, sec):.1f} GB/s)", file=out, flush=True)
            del host


# Selective scan over a sequence (prefill): the COREY page's kernel benchmark
# (Table 9, Table 17, Table 18): batch 1, dim 1024, d_state 16, L 4096 (8192),
# FP16 (BF16), static chunks of 512 tokens, one launch per chunk.
def scan_bytes(batch, dim, N, G, L):
    """Algorithmic HBM bytes of one scanned sequence: u, delta and out (16-bit)
    once, B and C (16-bit) once, the fp32 state read and written once, A, D and
    delta_bias once."""
    return 2 * 3 * batch * dim * L + 2 * 2 * batch * G * N * L + 8 * batch * dim * N + 4 * dim * (N + 2)


def scan_elements(batch, dim, N, L):
    """(request, channel, state, token) elements of one sequence."""
    return batch * dim * N * L


def run_scan(a):
    """ssu_scan on the page's shapes (configs from --scan), for every chunk in
    --chunks. Input sets (u, delta, B, C, out, state) rotate so that the sets
    together hold >= 768 MiB (cold HBM); K sequences captured in one HIP graph,
    median of 5 x 10 replays. warm_us_per_seq repeats one set instead, so its
    inputs stay in the Infinity Cache, as when the kernels before the scan have
    just written them (and as a harness that reuses one tensor measures). One
    line per (config, chunk, configuration)."""
    import torch

    import selective_state_update_amd as ssu

    out = open(a.out, "w") if a.out else sys.stdout
    print("config chunk launches us_per_seq ms_per_seq Mtokens_per_s GBps hbm_pct Gelem_per_s warm_us_per_seq tile "
          "batch", file=out, flush=True)
    chunks = [int(c) for c in a.chunks.split(",")]
    for k in [int(c) for c in a.scan.split(",")]:
        cfg = dict(si.SCAN_CONFIGS[k])
        name = cfg.pop("name")
        cfg.pop("chunk")
        if a.scan_batch:
            cfg["batch"] = a.scan_batch
            name += f", batch {a.scan_batch}"
        bs, dim, N, G, L = cfg["batch"], cfg["dim"], cfg["dstate"], cfg["ngroups"], cfg["seqlen"]
        nbytes = scan_bytes(bs, dim, N, G, L)
        K = max(2, -(-ROTATION_BYTES // nbytes))
        sets = []
        for i in range(K):
            p = si.make_scan_problem(**{**cfg, "seed": cfg["seed"] * 1000 + i}) if i < 2 else None
            if p is None:
                # further sets: the first two sets' inputs at new addresses (same values)
                sets.append({key: t.clone() for key, t in sets[i % 2].items()})
                continue
            dt = torch.float16 if p.io == "f16" else torch.bfloat16

            def dev(bits, dt=dt):
                return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).cuda()

            sets.append(dict(u=dev(p.u), delta=dev(p.delta), B=dev(p.B), C=dev(p.C),
                             A=torch.from_numpy(p.A).cuda(), D=torch.from_numpy(p.D).cuda(),
                             bias=torch.from_numpy(p.delta_bias).cuda(),
                             state=torch.from_numpy(p.state).cuda(),
                             out=torch.empty((bs, dim, L), dtype=dt, device="cuda")))
        args = [ssu.make_scan_args(s["u"], s["delta"], s["A"], s["B"], s["C"], s["state"], s["D"], s["bias"],
                                   True, s["out"])[0] for s in sets]
        tiles = range(len(ssu.scan_tiles())) if a.tile_sweep else [a.tile]
        for chunk in chunks:
            for tile in tiles:
                launches = -(-L // chunk) if chunk > 0 else 1
                calls = max(K, 8)
                side = torch.cuda.Stream()
                with torch.cuda.stream(side):
                    ssu.scan_launch(args[0], chunk, tile, stream=side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for i in range(calls):
                        ssu.scan_launch(args[i % K], chunk, tile, stream=side)
                g.replay()
                torch.cuda.synchronize()
                us = statistics.median([time_graph_on(g, 10, side) / (10 * calls) for _ in range(5)]) * 1e6
                del g
                # warm: the same set every call (its 25 MB stay in the Infinity Cache), as when the
                # activations were just written by the kernels before the scan
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for i in range(calls):
                        ssu.scan_launch(args[0], chunk, tile, stream=side)
                g.replay()
                torch.cuda.synchronize()
                warm = statistics.median([time_graph_on(g, 10, side) / (10 * calls) for _ in range(5)]) * 1e6
                del g
                gbs = nbytes / (us * 1e-6) / 1e9
                tname = (ssu.scan_tiles()[tile] if tile >= 0
                         else "default=" + ssu.scan_tiles()[ssu.scan_select_tile(args[0], chunk)])
                print(f"{k} {chunk} {launches} {us:.2f} {us / 1e3:.4f} {bs * L / us:.2f} {gbs:.1f} "
                      f"{100 * gbs / HBM_PEAK_GBS:.2f} {scan_elements(bs, dim, N, L) / (us * 1e3):.1f} {warm:.2f} "
                      f"{tname} {bs}", file=out, flush=True)
        if k == 1 and not a.no_cpu_baseline and not a.scan_batch:
            # the CPU oracle on one sequence of this workload, for context
            import oracle

            p = si.make_scan_problem(**cfg)
            threads = len(os.sched_getaffinity(0))
            t0 = time.perf_counter()
            oracle.get().scan(p.state.copy(), p.u, p.delta, p.A, p.B, p.C, p.D, p.delta_bias, io=p.io,
                              want_ref=False, nthreads=threads)
            print(f"# cpu oracle (fp64, {threads} threads): {(time.perf_counter() - t0) * 1e3:.1f} ms per sequence of "
                  f"{name}", file=out, flush=True)
        del sets, args
        torch.cuda.empty_cache()


def scan_launch_bytes(batch, dim, N, G, tokens):
    """Algorithmic HBM bytes of one scan launch over `tokens` tokens: its share
    of u, delta, out, B and C, plus the state read and written and A, D and
    delta_bias read once per launch."""
    return 2 * 3 * batch * dim * tokens + 2 * 2 * batch * G * N * tokens + 8 * batch * dim * N + 4 * dim * (N + 2)


def _copy_reference():
    """A plain device copy of known size (256 MiB read + 256 MiB written), cold,
    four times: what FETCH_SIZE / WRITE_SIZE read for it scales the counters."""
    import torch

    src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    bufs = [torch.empty_like(src) for _ in range(3)]  # evict src from the cache between copies
    for i in range(4):
        for b in bufs:
            b.fill_(float(i))
        torch.mul(src, 2.0, out=dst)  # one elementwise kernel: reads src once, writes dst once
    torch.cuda.synchronize()
    return src.numel() * 4


def run_scan_counters(a):
    """Eager scans for a rocprofv3 --pmc pass: `a.steps` sequences of scan
    config `a.scan` at the first of --chunks (default: its static chunk), over
    4 input sets of which each is evicted from the cache before reuse, then the
    reference copy."""
    import torch

    import selective_state_update_amd as ssu

    k = int(a.scan)
    cfg = dict(si.SCAN_CONFIGS[k])
    cfg.pop("name")
    chunk = cfg.pop("chunk")
    if a.chunks:
        chunk = int(a.chunks.split(",")[0])
    if a.scan_batch:
        cfg["batch"] = a.scan_batch
    dt = torch.float16 if cfg["io"] == "f16" else torch.bfloat16
    sets = []
    for i in range(4):
        p = si.make_scan_problem(**{**cfg, "seed": cfg["seed"] * 1000 + i})

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).cuda()

        t = dict(u=dev(p.u), delta=dev(p.delta), B=dev(p.B), C=dev(p.C), A=torch.from_numpy(p.A).cuda(),
                 D=torch.from_numpy(p.D).cuda(), bias=torch.from_numpy(p.delta_bias).cuda(),
                 state=torch.from_numpy(p.state).cuda())
        t["args"] = ssu.make_scan_args(t["u"], t["delta"], t["A"], t["B"], t["C"], t["state"], t["D"],
                                       t["bias"])[0]
        sets.append(t)
    flush = torch.empty(3 * LLC_BYTES // 4, dtype=torch.float32, device="cuda")
    for i in range(a.steps):
        flush.fill_(float(i))  # evicts the previous sequence's inputs from the Infinity Cache
        ssu.scan_launch(sets[i % 4]["args"], chunk, a.tile)
    torch.cuda.synchronize()
    n = _copy_reference()
    print(f"# scan counters pass: {a.steps} sequences of config {k} (batch {cfg['batch']}) at chunk {chunk}, "
          f"4 copies of {n} bytes", flush=True)


def run_counters(a):
    """Eager calls for a rocprofv3 --pmc pass: `a.steps` headline calls rotating
    over the slot sets, then a plain device copy of a known size (256 MiB read
    + 256 MiB written) to scale the counters."""
    import torch

    import selective_state_update_amd as ssu

    w = WORKLOADS[a.config]
    H, P, N, G, bs = w["H"], w["P"], w["N"], w["G"], w["batch"]
    rot = Rotation(H, P, N, G, bs, seed=a.config)
    h = ssu.Handle(H, P, N, G, True, a.tile)
    args = rot.args(h)
    for i in range(a.steps):
        h.launch(args[i % len(args)])
    torch.cuda.synchronize()
    n = _copy_reference()
    print(f"# counters pass: {a.steps} ssu calls, 4 copies of {n} bytes", flush=True)


def _load_counter(dirpath, counter):
    """(kernel name, value) rows of one counter from rocprofv3 --pmc CSV output."""
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


SCAN_COUNTER_PROFILE = os.path.join(ROOT, "profiles", "ssu_scan_dim1024_L4096_f16_chunk512_counters.md")


def summarize_scan_counters(a):
    """Counter summary for the scan kernel (see run_scan_counters)."""
    fetch_dir, write_dir = a.summarize_scan_counters.split(",")
    fetch, write = _load_counter(fetch_dir, "FETCH_SIZE"), _load_counter(write_dir, "WRITE_SIZE")
    def is_scan(k):
        return any(f"ssu_scan_{kind}_kernel" in k for kind in ("direct", "staged", "paired"))

    fs = [v for k, v in fetch if is_scan(k)]
    ws = [v for k, v in write if is_scan(k)]
    kernels = sorted({k for k, v in fetch if is_scan(k)})
    fc = [v for k, v in fetch if "MulFunctor" in k]
    wc = [v for k, v in write if "MulFunctor" in k]
    if not fs or not ws or not fc or not wc:
        raise SystemExit("no counter rows found")
    copy_bytes = 64 * 1024 * 1024 * 4
    f_scale = copy_bytes / (statistics.median(fc) * 1024)
    w_scale = copy_bytes / (statistics.median(wc) * 1024)
    k = int(a.scan)
    c = si.SCAN_CONFIGS[k]
    per_launch = scan_launch_bytes(c["batch"], c["dim"], c["dstate"], c["ngroups"], c["chunk"])
    f_b = statistics.median(fs) * 1024 * f_scale
    w_b = statistics.median(ws) * 1024 * w_scale
    cmd = f"python3 bench.py --scan {k} --scan-counters --steps {a.steps}"
    text = f"""# rocprofv3 HBM counters: the selective scan, {c['name']}

Commands (run from the repository root on one MI355X):

    rocprofv3 --pmc FETCH_SIZE -f csv -d {a.fetch_dir_name} -o run -- {cmd}
    rocprofv3 --pmc WRITE_SIZE -f csv -d {a.write_dir_name} -o run -- {cmd}
    python3 bench.py --scan {k} --summarize-scan-counters {a.fetch_dir_name},{a.write_dir_name} --write-profile

Counters are KiB per dispatch, scaled by the ratio (known bytes / counter) of a
plain device copy of 268435456 bytes read + 268435456 written in the same run.
Each dispatch is one chunk of {c['chunk']} tokens; the Infinity Cache is
flushed between sequences.

- scan_code_digest: `{scan_source_digest()}`
- kernel: `{"`, `".join(kernels)}`
- scan_dispatches: {len(fs)}
- fetch_kib_median: {statistics.median(fs):.1f}
- write_kib_median: {statistics.median(ws):.1f}
- fetch_scale: {f_scale:.4f}
- write_scale: {w_scale:.4f}
- fetch_bytes_per_launch: {f_b:.0f}
- write_bytes_per_launch: {w_b:.0f}
- traffic_bytes_per_launch: {f_b + w_b:.0f}
- algorithmic_bytes_per_launch: {per_launch}
- traffic_over_algorithmic: {(f_b + w_b) / per_launch:.4f}
"""
    if a.write_profile:
        with open(SCAN_COUNTER_PROFILE, "w") as f:
            f.write(text)
    print(text)


def summarize_counters(a):
    """Read rocprofv3 --pmc CSV output (FETCH_SIZE and WRITE_SIZE runs) and write
    the counter summary that the JSON line's roofline.traffic comes from."""
    load = _load_counter
    fetch_dir, write_dir = a.summarize_counters.split(",")
    fetch = load(fetch_dir, "FETCH_SIZE")
    write = load(write_dir, "WRITE_SIZE")
    if not fetch or not write:
        raise SystemExit("no counter rows found")

    def split(rows):
        ssu_v = [v for k, v in rows if "ssu_decode_kernel" in k]
        copy_v = [v for k, v in rows if "MulFunctor" in k]
        return ssu_v, copy_v

    fs, fc = split(fetch)
    ws, wc = split(write)
    copy_bytes = 64 * 1024 * 1024 * 4
    # counters are in KiB per dispatch; scale by what a copy of known size reads
    f_scale = copy_bytes / (statistics.median(fc) * 1024) if fc else 1.0
    w_scale = copy_bytes / (statistics.median(wc) * 1024) if wc else 1.0
    w = WORKLOADS[a.config]
    nbytes = algorithmic_bytes(w["H"], w["P"], w["N"], w["G"], w["batch"])
    f_b = statistics.median(fs) * 1024 * f_scale
    w_b = statistics.median(ws) * 1024 * w_scale
    text = f"""# rocprofv3 HBM counters: ssu_decode_kernel, H{w['H']} P{w['P']} N{w['N']} batch {w['batch']}

Commands (run from the repository root on one MI355X):

    rocprofv3 --pmc FETCH_SIZE -f csv -d {a.fetch_dir_name} -o run -- python3 bench.py --counters --steps {a.steps}
    rocprofv3 --pmc WRITE_SIZE -f csv -d {a.write_dir_name} -o run -- python3 bench.py --counters --steps {a.steps}
    python3 bench.py --summarize-counters {a.fetch_dir_name},{a.write_dir_name} --steps {a.steps} --write-profile

Counters are KiB per dispatch. Each is scaled by the ratio (known bytes / counter)
measured on a plain device copy of 268435456 bytes read + 268435456 written in the
same run.

- kernel_code_digest: `{source_digest()}`
- ssu_dispatches: {len(fs)}
- fetch_kib_median: {statistics.median(fs):.1f}
- write_kib_median: {statistics.median(ws):.1f}
- copy_fetch_kib_median: {statistics.median(fc) if fc else float('nan'):.1f}
- copy_write_kib_median: {statistics.median(wc) if wc else float('nan'):.1f}
- fetch_scale: {f_scale:.4f}
- write_scale: {w_scale:.4f}
- fetch_bytes_per_launch: {f_b:.0f}
- write_bytes_per_launch: {w_b:.0f}
- traffic_bytes_per_launch: {f_b + w_b:.0f}
- algorithmic_bytes_per_launch: {nbytes}
- traffic_over_algorithmic: {(f_b + w_b) / nbytes:.4f}
"""
    if a.write_profile:
        with open(COUNTER_PROFILE, "w") as f:
            f.write(text)
    print(text)


def run_floors(a):
    """Per-call floors of the decode step at H16 P64 N128, at each batch of
    --batches (default 8 and 128), same rotation and graph method as the
    headline (cold sets, max(20, K) launches per graph, median of 5 x 10
    replays):
      (1) a graph launch of a 1-element kernel: the launch floor;
      (2) ssu_update with every slot id padding: the launch, the id reads and
          the small operands, no state traffic;
      (3) ssu_update on one request (512 KiB of state): the launch plus one
          dependent idx -> state round trip;
      (4) a device copy of the call's state bytes (read and written,
          contiguous, rotating buffers over >= 768 MiB): the bare stream;
      (5) ssu_update at the batch."""
    import torch

    import selective_state_update_amd as ssu

    out = open(a.out, "w") if a.out else sys.stdout
    batches = [int(b) for b in (a.batches or "8,128").split(",")]
    H, P, N, G = 16, 64, 128, 1
    print("batch us_per_call what", file=out, flush=True)

    def timed(fn, calls):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(calls):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        us = statistics.median([time_graph(g, 10) / (10 * calls) for _ in range(5)]) * 1e6
        del g
        return us

    for bs in batches:
        rot = Rotation(H, P, N, G, bs, seed=9100 + bs)
        one = Rotation(H, P, N, G, 1, seed=9200 + bs)
        calls = max(20, rot.K)
        h = ssu.Handle(H, P, N, G, True, a.tile)
        args = rot.args(h)
        pad = torch.full((bs,), -1, dtype=torch.int32, device="cuda")
        pad_args = [h.make_args(rot.pool, pad, s["x"], s["B"], s["C"], s["dt"], rot.A, rot.D, rot.dt_bias, s["out"])
                    for s in rot.sets]
        one_args = one.args(h)
        nbytes = bs * H * P * N * 4
        pairs = max(2, -(-ROTATION_BYTES // (2 * nbytes)))
        bufs = [(torch.empty(nbytes // 4, device="cuda"), torch.empty(nbytes // 4, device="cuda"))
                for _ in range(pairs)]
        tiny = torch.zeros(1, device="cuda")
        rows = [
            ("launch of a 1-element kernel", lambda i: tiny.add_(1.0), calls),
            ("ssu_update, every slot id padding (no state traffic)", lambda i: h.launch(pad_args[i % rot.K]), calls),
            ("ssu_update on one request (512 KiB of state)", lambda i: h.launch(one_args[i % one.K]),
             max(20, one.K)),
            (f"device copy of the call's state bytes ({nbytes >> 20} MiB read + written, {pairs} rotating pairs)",
             lambda i: bufs[i % pairs][1].copy_(bufs[i % pairs][0]), max(20, pairs)),
            (f"ssu_update ({ssu.tiles()[h.selected_tile(bs)]['name']})", lambda i: h.launch(args[i % rot.K]), calls),
        ]
        for what, fn, n in rows:
            us = timed(fn, n)
            print(f"{bs} {us:.3f} {what}", file=out, flush=True)
        del rot, one, bufs
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=3, choices=sorted(WORKLOADS))
    ap.add_argument("--tile", type=int, default=-1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--heads", default="")
    ap.add_argument("--batches", default="")
    ap.add_argument("--out", default="")
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--tile-sweep", action="store_true")
    ap.add_argument("--shapes", default="", help="comma list of HxPxNxGxBATCH decode shapes")
    ap.add_argument("--copy-ceiling", action="store_true")
    ap.add_argument("--floors", action="store_true", help="per-call floors of the decode step (--batches)")
    ap.add_argument("--tokens", default="", help="comma list of tokens per call (ssu_update_tokens)")
    ap.add_argument("--copy-blocks", default="", help="comma list of request counts (ssu_copy_blocks)")
    ap.add_argument("--scan", default="", help="comma list of scan configs (ssu_scan), e.g. 1,2,3")
    ap.add_argument("--chunks", default="512", help="comma list of scan chunk sizes (0: one launch)")
    ap.add_argument("--scan-batch", type=int, default=0, help="override the scan workload's batch (requests)")
    ap.add_argument("--scan-counters", action="store_true", help="eager scans for rocprofv3 --pmc")
    ap.add_argument("--summarize-scan-counters", default="")
    ap.add_argument("--summarize-counters", default="")
    ap.add_argument("--write-profile", action="store_true")
    ap.add_argument("--fetch-dir-name", default="pmc/fetch", help="FETCH_SIZE output directory (for the summary text)")
    ap.add_argument("--write-dir-name", default="pmc/write", help="WRITE_SIZE output directory (for the summary text)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU: selective_state_update exchanges nothing between GPUs (each "
              "GPU holds its heads' or requests' share), so only --gpus 1 is measured.", file=sys.stderr)
        sys.exit(2)
    if a.summarize_counters:
        summarize_counters(a)
    elif a.summarize_scan_counters:
        summarize_scan_counters(a)
    elif a.scan and a.scan_counters:
        run_scan_counters(a)
    elif a.scan:
        run_scan(a)
    elif a.counters:
        run_counters(a)
    elif a.shapes:
        run_shapes(a)
    elif a.tile_sweep:
        run_tile_sweep(a)
    elif a.copy_ceiling:
        run_copy_ceiling(a)
    elif a.floors:
        run_floors(a)
    elif a.tokens:
        run_tokens(a)
    elif a.copy_blocks:
        run_copy_blocks(a)
    elif a.sweep:
        run_sweep(a)
    else:
        run_bench(a)


if __name__ == "__main__":
    main()
