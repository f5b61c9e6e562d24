"""Seeded synthetic inputs for the Mamba2 decode-step selective_state_update.

This module draws random numbers and encodes them in the storage formats the
decode step consumes (fp32 state pool, bf16 activations, fp32 per-head
parameters, int32 slot indices). It holds none of the update's arithmetic and
is the only code shared by the CPU oracle harness, the GPU tests and the
benchmark.

The shapes and distributions follow the kernel workload of sglang PR #41223
("[Perf] Mamba2 selective_state_update up to 2x faster on B200 via 8x1 launch
config for dstate 128"), section "Kernel measurement": a state pool
[pool, H, 64, 128] fp32 addressed through random state_batch_indices, x
[bs, H, 64] and B/C [bs, 1, 128] as views into one packed bf16 tensor, and
dt/A/D/dt_bias broadcast per head. Section "Model" of the same page gives the
per-rank shape (16 heads, headdim 64, dstate 128, fp32 SSM cache).

Recipe (seeded, deterministic):
  * every non-pool input comes from ``numpy.random.Generator(PCG64(seed))``
    drawn in this order: xBC, dt, dt_bias, A, D, idx;
  * the state pool comes from its own stream, ``PCG64([seed, 1])`` on the host,
    or ``torch.Generator`` seeded with ``seed`` when drawn on a GPU (large pools);
  * pool  : fp32 ~ N(0, 1);
  * xBC   : bf16 = RNE(N(0, 1)), one row [x (H*P) | B (G*N) | C (G*N)] per request;
  * dt    : bf16 = RNE(N(0, 1)), one value per (request, head);
  * dt_bias: fp32 = log(expm1(y)), y ~ U(1e-3, 0.1), per head (so that the
    softplus of the bias alone lies in [1e-3, 0.1]);
  * A     : fp32 = -exp(U(0, log 16)), per head;
  * D     : fp32 ~ N(0, 1), per head;
  * idx   : int32, distinct, random order, drawn from range(pool_slots).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Problem",
    "make_problem",
    "bf16_bits",
    "bf16_values",
    "rotation_sets",
    "sweep_points",
    "sweep_seed",
    "CONFIGS",
    "ScanProblem",
    "make_scan_problem",
    "io_bits",
    "io_values",
    "SCAN_CONFIGS",
]


def bf16_bits(a) -> np.ndarray:
    """Encode float values as bf16 bit patterns (uint16), round-to-nearest-even.

    Used only to store drawn inputs in bf16; the values drawn here are finite.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_values(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Problem:
    """One decode step's inputs, in storage form.

    Arrays are numpy. ``xbc`` is the packed activation tensor; ``x``, ``B`` and
    ``C`` are strided views into it.
    """

    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    batch: int
    pool_slots: int
    dt_softplus: bool
    seed: int
    pool: np.ndarray | None  # float32 [pool_slots, H, P, N] (None: drawn on a device)
    xbc: np.ndarray  # uint16 [batch, H*P + 2*G*N]
    dt: np.ndarray  # uint16 [batch, H]
    dt_bias: np.ndarray  # float32 [H]
    A: np.ndarray  # float32 [H]
    D: np.ndarray  # float32 [H]
    idx: np.ndarray  # int32 [batch]
    extra: dict = field(default_factory=dict)

    @property
    def x(self) -> np.ndarray:
        H, P = self.nheads, self.headdim
        return self.xbc[:, : H * P].reshape(self.batch, H, P)

    @property
    def B(self) -> np.ndarray:
        o, GN = self.nheads * self.headdim, self.ngroups * self.dstate
        return self.xbc[:, o : o + GN].reshape(self.batch, self.ngroups, self.dstate)

    @property
    def C(self) -> np.ndarray:
        o, GN = self.nheads * self.headdim + self.ngroups * self.dstate, self.ngroups * self.dstate
        return self.xbc[:, o : o + GN].reshape(self.batch, self.ngroups, self.dstate)


def draw_pool(pool_slots: int, H: int, P: int, N: int, seed: int) -> np.ndarray:
    """fp32 ~ N(0,1) state pool from its own host stream."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    return rng.standard_normal((pool_slots, H, P, N), dtype=np.float32)


def draw_pool_on_device(pool, seed: int):
    """Fill a torch tensor (any device) with fp32 ~ N(0,1) from torch's seeded generator."""
    import torch

    g = torch.Generator(device=pool.device)
    g.manual_seed(int(seed))
    pool.normal_(0.0, 1.0, generator=g)
    return pool


def make_problem(
    H: int,
    P: int = 64,
    N: int = 128,
    G: int = 1,
    batch: int = 4,
    pool_slots: int | None = None,
    seed: int = 0,
    dt_softplus: bool = True,
    host_pool: bool = True,
    idx: np.ndarray | None = None,
) -> Problem:
    """Draw one decode step's inputs following the recipe in the module docstring."""
    if pool_slots is None:
        pool_slots = 2 * batch
    if batch > pool_slots and idx is None:
        raise ValueError("need pool_slots >= batch for distinct indices")
    pool = draw_pool(pool_slots, H, P, N, seed) if host_pool else None
    rng = np.random.Generator(np.random.PCG64(seed))
    row = H * P + 2 * G * N
    xbc = bf16_bits(rng.standard_normal((batch, row), dtype=np.float32))
    dt = bf16_bits(rng.standard_normal((batch, H), dtype=np.float32))
    y = rng.uniform(1e-3, 0.1, size=H)
    dt_bias = np.log(np.expm1(y)).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    if idx is None:
        idx = rng.permutation(pool_slots)[:batch].astype(np.int32)
    else:
        idx = np.asarray(idx, dtype=np.int32)
    return Problem(
        nheads=H, headdim=P, dstate=N, ngroups=G, batch=batch, pool_slots=pool_slots,
        dt_softplus=dt_softplus, seed=seed, pool=pool, xbc=xbc, dt=dt, dt_bias=dt_bias,
        A=A, D=D, idx=idx, extra={"softplus_of_bias_target": y},
    )


def rotation_sets(state_bytes_per_call: int, batch: int, min_total_bytes: int, seed: int):
    """Disjoint slot sets for cold-cache timing.

    K = ceil(min_total_bytes / state_bytes_per_call) sets of ``batch`` slots,
    carved from one random permutation of K*batch slots (the pool holds exactly
    K*batch slots). Returns (K, int32 array [K, batch]).
    """
    K = max(1, -(-min_total_bytes // state_bytes_per_call))
    rng = np.random.Generator(np.random.PCG64([seed, 2]))
    perm = rng.permutation(K * batch).astype(np.int32)
    return K, perm.reshape(K, batch)


def sweep_points():
    """The (heads, batch) grid of the bitwise sweep in sglang PR #41223
    ("Kernel measurement"): heads {8,16,32,64,128} x batch {1..64, then every 8
    up to 1024}, 920 points."""
    batches = list(range(1, 65)) + list(range(72, 1025, 8))
    return [(H, bs) for H in (8, 16, 32, 64, 128) for bs in batches]


def sweep_seed(H: int, bs: int) -> int:
    return 1000 * H + bs


# The five workloads (shapes only; seeds are the config number).
CONFIGS = {
    0: dict(name="tiny H2 P64 N128 bs4 pool8", H=2, P=64, N=128, G=1, batch=4, pool_slots=8, seed=0),
    1: dict(name="H16 P64 N128 bs8", H=16, P=64, N=128, G=1, batch=8, seed=1),
    2: dict(name="H16 P64 N128 bs128", H=16, P=64, N=128, G=1, batch=128, seed=2),
    3: dict(name="H16 P64 N128 bs512", H=16, P=64, N=128, G=1, batch=512, seed=3),
}


# ---------------------------------------------------------------------------
# Selective scan over a sequence (prefill)
#
# Shapes and distributions follow the selective_scan_fn benchmark of the COREY
# page (COREY: Entropy-Guided Runtime Chunk Scheduling for Selective Scan
# Kernels, Table 9, Table 17 and Table 18): batch 1, dim 1024 channels,
# d_state 16, sequence 4096 (also 8192), FP16 (also BF16) activations drawn
# standard normal, static chunks of 512 tokens. The page does not give the
# parameter distributions; the recipe below takes the usual Mamba ones.
#
# Recipe (seeded, deterministic), ``numpy.random.Generator(PCG64([seed, 3]))``
# drawn in this order:
#   * u, delta : io = RNE(N(0, 1)), [batch, dim, L];
#   * B, C     : io = RNE(N(0, 1)), [batch, G, dstate, L];
#   * A        : fp32 = -(n + 1) * U(0.5, 1.5), [dim, dstate] (a jittered
#                -1, -2, ..., -dstate ladder per channel);
#   * D        : fp32 ~ U(0.5, 1.5), [dim];
#   * delta_bias: fp32 = log(expm1(y)), y ~ U(1e-3, 0.1), [dim];
#   * state    : fp32 zeros (a fresh sequence), or ~ N(0, 1) on request.
# io is fp16 or bf16, rounded to nearest even.
# ---------------------------------------------------------------------------


def io_bits(a, io: str) -> np.ndarray:
    """Encode float values as fp16 or bf16 bit patterns (uint16), RNE."""
    if io == "bf16":
        return bf16_bits(a)
    if io == "f16":
        return np.ascontiguousarray(np.asarray(a, dtype=np.float32).astype(np.float16)).view(np.uint16)
    raise ValueError(f"io must be 'f16' or 'bf16', not {io!r}")


def io_values(bits, io: str) -> np.ndarray:
    """Decode fp16 or bf16 bit patterns to float32 (exact)."""
    if io == "bf16":
        return bf16_values(bits)
    if io == "f16":
        return np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.float16).astype(np.float32)
    raise ValueError(f"io must be 'f16' or 'bf16', not {io!r}")


@dataclass
class ScanProblem:
    """A selective scan's inputs, in storage form (numpy arrays)."""

    batch: int
    dim: int
    dstate: int
    ngroups: int
    seqlen: int
    io: str
    delta_softplus: bool
    seed: int
    u: np.ndarray          # io bits [batch, dim, L]
    delta: np.ndarray      # io bits [batch, dim, L]
    B: np.ndarray          # io bits [batch, G, dstate, L]
    C: np.ndarray          # io bits [batch, G, dstate, L]
    A: np.ndarray          # fp32 [dim, dstate]
    D: np.ndarray          # fp32 [dim]
    delta_bias: np.ndarray  # fp32 [dim]
    state: np.ndarray      # fp32 [batch, dim, dstate]


def make_scan_problem(batch: int, dim: int, dstate: int, seqlen: int, ngroups: int = 1, io: str = "f16",
                      seed: int = 0, zero_state: bool = True, delta_softplus: bool = True) -> ScanProblem:
    """Draw a selective scan's inputs following the recipe above."""
    if dim % ngroups:
        raise ValueError("dim must be a multiple of ngroups")
    rng = np.random.Generator(np.random.PCG64([seed, 3]))
    L = seqlen
    u = io_bits(rng.standard_normal((batch, dim, L), dtype=np.float32), io)
    delta = io_bits(rng.standard_normal((batch, dim, L), dtype=np.float32), io)
    B = io_bits(rng.standard_normal((batch, ngroups, dstate, L), dtype=np.float32), io)
    C = io_bits(rng.standard_normal((batch, ngroups, dstate, L), dtype=np.float32), io)
    A = (-(np.arange(dstate, dtype=np.float64) + 1.0) * rng.uniform(0.5, 1.5, size=(dim, dstate))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=dim).astype(np.float32)
    y = rng.uniform(1e-3, 0.1, size=dim)
    delta_bias = np.log(np.expm1(y)).astype(np.float32)
    if zero_state:
        state = np.zeros((batch, dim, dstate), dtype=np.float32)
    else:
        state = rng.standard_normal((batch, dim, dstate), dtype=np.float32)
    return ScanProblem(batch=batch, dim=dim, dstate=dstate, ngroups=ngroups, seqlen=L, io=io,
                       delta_softplus=delta_softplus, seed=seed, u=u, delta=delta, B=B, C=C, A=A, D=D,
                       delta_bias=delta_bias, state=state)


# Scan workloads: 1-3 are the page's benchmark shapes (static chunk 512);
# 0 is a small case the oracle finishes at once, with a ragged length.
SCAN_CONFIGS = {
    0: dict(name="scan b2 dim64 N16 G2 L1000 f16", batch=2, dim=64, dstate=16, ngroups=2, seqlen=1000,
            io="f16", chunk=512, seed=10),
    1: dict(name="scan b1 dim1024 N16 L4096 f16 chunk512", batch=1, dim=1024, dstate=16, ngroups=1,
            seqlen=4096, io="f16", chunk=512, seed=11),
    2: dict(name="scan b1 dim1024 N16 L4096 bf16 chunk512", batch=1, dim=1024, dstate=16, ngroups=1,
            seqlen=4096, io="bf16", chunk=512, seed=12),
    3: dict(name="scan b1 dim1024 N16 L8192 f16 chunk512", batch=1, dim=1024, dstate=16, ngroups=1,
            seqlen=8192, io="f16", chunk=512, seed=13),
}
