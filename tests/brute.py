"""Independent pure-Python fp64 brute force of the decode step, for tiny shapes.

Written separately from the C oracle and in a different form, to pin it:
softplus as log(1 + e^u) (with the asymptote for large u), the output sum as
``math.fsum`` (correctly rounded), fp32 rounding through ``struct`` and bf16
rounding by comparing the dropped half-word against the halfway point.
Per (request b, head h): S' = S*a + delta*x[p]*B[n] with a = exp(A*delta),
y[p] = sum_n S'[p,n]*C[n] + D*x[p], group g(h) = h // (H // G).
"""
from __future__ import annotations

import math
import struct


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16_bits_of_f32(v: float) -> int:
    w = struct.unpack("<I", struct.pack("<f", v))[0]
    hi, lo = w >> 16, w & 0xFFFF
    if lo > 0x8000 or (lo == 0x8000 and (hi & 1)):
        hi += 1
    return hi & 0xFFFF


def _softplus(u: float) -> float:
    if u > 40.0:
        return u + math.exp(-u)
    return math.log(1.0 + math.exp(u)) if u > -30.0 else math.exp(u)


def step(pool, idx, x, B, C, dt, A, dt_bias, D, softplus=True):
    """pool: nested lists [slots][H][P][N] of floats (a copy is returned updated in fp64);
    idx [bs]; x [bs][H][P] bf16 bits; B, C [bs][G][N] bf16 bits; dt [bs][H] bf16 bits;
    A, dt_bias, D: [H] floats (dt_bias / D may be None).

    Returns (new_pool_fp64, y [bs][H][P], out_bits [bs][H][P]).
    """
    bs, H = len(x), len(x[0])
    P = len(x[0][0])
    G, N = len(B[0]), len(B[0][0])
    new = [[[list(row) for row in head] for head in slot] for slot in pool]
    y = [[[0.0] * P for _ in range(H)] for _ in range(bs)]
    out = [[[0] * P for _ in range(H)] for _ in range(bs)]
    for b in range(bs):
        s = int(idx[b])
        if s < 0 or s >= len(pool):
            continue
        for h in range(H):
            g = h // (H // G)
            u = _bf16(dt[b][h]) + (float(dt_bias[h]) if dt_bias is not None else 0.0)
            delta = _softplus(u) if softplus else u
            decay = math.exp(float(A[h]) * delta)
            d = float(D[h]) if D is not None else 0.0
            for p in range(P):
                xp = _bf16(x[b][h][p])
                terms = []
                for n in range(N):
                    v = float(pool[s][h][p][n]) * decay + delta * xp * _bf16(B[b][g][n])
                    new[s][h][p][n] = v
                    terms.append(v * _bf16(C[b][g][n]))
                terms.append(d * xp)
                yy = math.fsum(terms)
                y[b][h][p] = yy
                out[b][h][p] = _bf16_bits_of_f32(_f32(yy))
    return new, y, out


# --------------------------------------------------------------------------- #
# Selective scan over a sequence, in explicit-sum form.
#
# Unrolling the recurrence h_t = a_t h_{t-1} + Delta_t u_t B_t gives, with the
# decay over tokens s+1..t written as one exponential of the summed steps,
#   h_t[n] = exp(A[n] * sum_{r<=t} Delta_r) h_{-1}[n]
#            + sum_{s<=t} exp(A[n] * sum_{s<r<=t} Delta_r) Delta_s u_s B_s[n]
#   y_t    = sum_n C_t[n] h_t[n] + D u_t
# Each term is evaluated directly (quadratic in the length), sums with
# math.fsum, fp16 decoded by struct's binary16 format.
# --------------------------------------------------------------------------- #
def _f16(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))[0]


def _io(bits: int, io: str) -> float:
    return _f16(bits) if io == "f16" else _bf16(bits)


def scan(state, u, delta, A, B, C, D, delta_bias, softplus, io, want_tau=False):
    """state [bs][dim][N] floats; u, delta [bs][dim][L] io bits; B, C
    [bs][G][N][L] io bits; A [dim][N]; D, delta_bias [dim] or None.

    Returns (h_final [bs][dim][N], y [bs][dim][L]) in fp64, and with
    ``want_tau`` also tau [bs][dim][L] = sum_n |C_t[n] h_t[n]| + |D u_t|.
    """
    bs, dim, L = len(u), len(u[0]), len(u[0][0])
    G, N = len(B[0]), len(B[0][0])
    h_out = [[[0.0] * N for _ in range(dim)] for _ in range(bs)]
    y_out = [[[0.0] * L for _ in range(dim)] for _ in range(bs)]
    tau_out = [[[0.0] * L for _ in range(dim)] for _ in range(bs)]
    for b in range(bs):
        for d in range(dim):
            g = d // (dim // G)
            bias = float(delta_bias[d]) if delta_bias is not None else 0.0
            steps = []
            for t in range(L):
                v = _io(delta[b][d][t], io) + bias
                steps.append(_softplus(v) if softplus else v)
            us = [_io(u[b][d][t], io) for t in range(L)]
            dd = float(D[d]) if D is not None else 0.0

            def h_at(t, n):
                an = float(A[d][n])
                terms = [math.exp(an * math.fsum(steps[: t + 1])) * float(state[b][d][n])]
                for s in range(t + 1):
                    decay = math.exp(an * math.fsum(steps[s + 1 : t + 1]))
                    terms.append(decay * steps[s] * us[s] * _io(B[b][g][n][s], io))
                return math.fsum(terms)

            for t in range(L):
                terms = [_io(C[b][g][n][t], io) * h_at(t, n) for n in range(N)] + [dd * us[t]]
                y_out[b][d][t] = math.fsum(terms)
                tau_out[b][d][t] = math.fsum(abs(v) for v in terms)
            for n in range(N):
                h_out[b][d][n] = h_at(L - 1, n) if L > 0 else float(state[b][d][n])
    return (h_out, y_out, tau_out) if want_tau else (h_out, y_out)
