"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the mathematics or a library routine fixes. They are
run against the real oracle (tests/test_oracle_pins.py) and against copies of
it with planted mistakes (tests/test_oracle_mutants.py), which must each fail
at least one pin.

What pins what:
  * discretisation  -- softplus closed forms and numpy.logaddexp; the dt_bias
    generator's inverse softplus; exp(A * 0) = 1;
  * bf16 rounding   -- torch's float32 -> bfloat16 conversion (ties, overflow,
    subnormals, signed zero, NaN);
  * rank-1 update   -- numpy a*S + delta*outer(x, B) in fp64; write-back is the
    fp32 rounding of it;
  * output          -- numpy S' @ C + D*x (matrix-vector product) in fp64;
  * gather          -- untouched slots bitwise unchanged; permuting requests
    permutes outputs; padding entries skipped; duplicates rejected;
  * special cases   -- dt = 0 (softplus off, no bias) leaves the state unchanged;
    A -> -1e9 collapses the state to delta*x*B; B = 0 is a pure decay; C = 0
    gives out = bf16(D*x) exactly;
  * groups          -- g(h) = h // (H/G) checked head by head;
  * K steps         -- the fp64 scan equals the closed form of the unrolled
    recurrence, and K single steps with fp32 storage stay within rounding of it;
  * everything      -- an independent pure-Python brute force (tests/brute.py).
  * block copy      -- numpy fancy-index assignment; skip, no-op and rejection
    rules; strided blocks.
Selective scan over a sequence:
  * fp16            -- all 65536 patterns decode to numpy's float16; fp32 ->
    fp16 rounding matches numpy (ties, subnormals, overflow, inf, NaN);
  * the scan        -- an explicit-sum brute force (decays as one exponential
    of summed steps, tests/brute.py); the geometric series for constant
    inputs; A = 0 gives numpy.cumsum; A -> -1e30 forgets everything; zero
    steps leave the state unchanged; two pieces with the state carried equal
    the whole; the error scales bound an fp32 numpy scan (short and long
    memory).
"""
from __future__ import annotations

import math

import numpy as np

import ssu_inputs as si

from . import brute


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _small(H=3, P=8, N=16, G=1, bs=3, slots=7, seed=11, softplus=True):
    return si.make_problem(H, P, N, G, bs, slots, seed, dt_softplus=softplus)


def _run(o, p, pool=None, **kw):
    pool = p.pool.copy() if pool is None else pool
    args = dict(dt_bias=p.dt_bias, D=p.D, dt_softplus=p.dt_softplus)
    args.update(kw)
    r = o.run(pool, p.idx, p.x, p.B, p.C, p.dt, args.pop("A", p.A), **args)
    return pool, r


def _np_delta(dt_bits, bias, softplus):
    u = si.bf16_values(dt_bits).astype(np.float64) + np.asarray(bias, dtype=np.float64)
    return np.logaddexp(0.0, u) if softplus else u


# --------------------------------------------------------------------------- #
def pin_softplus_closed_forms(o):
    assert abs(o.softplus(0.0) - math.log(2.0)) <= 1e-16
    for u in np.concatenate([np.linspace(-50, 50, 201), [-700.0, 1000.0, 1e-300, -1e-300]]):
        want = np.logaddexp(0.0, u)
        got = o.softplus(u)
        assert abs(got - want) <= 4e-16 * max(abs(want), 1e-300), (u, got, want)
    # the dt_bias generator's inverse softplus: softplus(log(expm1(y))) = y
    y = _rng(5).uniform(1e-3, 0.1, size=64)
    for yy in y:
        got = o.softplus(float(np.log(np.expm1(yy))))
        assert abs(got - yy) <= 1e-14 * yy, (yy, got)
    # discretisation: delta = u (softplus off), a = exp(A * delta); A*0 -> a = 1
    d, a = o.discretize(0.0, 0.0, -3.5, softplus=False)
    assert d == 0.0 and a == 1.0
    d, a = o.discretize(0.25, 0.5, 0.0, softplus=True)
    assert a == 1.0 and abs(d - np.logaddexp(0.0, 0.75)) <= 1e-16
    for dt, bias, A, sp in ((0.3, -0.1, -2.0, False), (-1.5, 0.05, -7.25, True), (4.0, 0.02, -16.0, True)):
        d, a = o.discretize(dt, bias, A, softplus=sp)
        dd = np.logaddexp(0.0, dt + bias) if sp else dt + bias
        assert abs(d - dd) <= 1e-15 * abs(dd)
        assert abs(a - math.exp(A * dd)) <= 1e-15 * math.exp(A * dd)


def pin_bf16_rounding(o):
    import torch

    rng = _rng(6)
    vals = [rng.standard_normal(2000).astype(np.float32),
            (rng.standard_normal(500) * 1e-39).astype(np.float32),    # subnormals
            (rng.standard_normal(500) * 1e30).astype(np.float32)]
    # exact ties: low half-word 0x8000, even and odd kept halves
    hi = rng.integers(0, 0x7F7F, size=400, dtype=np.uint32)
    vals.append(((hi << 16) | 0x8000).view(np.float32))
    vals.append((((hi << 16) | 0x8000) | 0x80000000).view(np.float32))
    vals.append(np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, -3.4e38,
                          np.finfo(np.float32).max, 1.0, -1.0, 2 ** -133, -(2 ** -140)],
                         dtype=np.float32))
    f = np.concatenate(vals)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.bf16_rne(f)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]
    nan = o.bf16_rne(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def pin_rank1_update(o):
    for seed, softplus in ((21, True), (22, False)):
        p = _small(seed=seed, softplus=softplus)
        before = p.pool.copy()
        pool, r = _run(o, p)
        delta = _np_delta(p.dt, p.dt_bias[None, :], softplus)
        for b in range(p.batch):
            for h in range(p.nheads):
                S0 = before[p.idx[b], h].astype(np.float64)
                a = np.exp(np.float64(p.A[h]) * delta[b, h])
                x = si.bf16_values(p.x[b, h]).astype(np.float64)
                Bv = si.bf16_values(p.B[b, 0]).astype(np.float64)
                want = a * S0 + delta[b, h] * np.outer(x, Bv)
                got = r["state"][b, h]
                assert np.allclose(got, want, rtol=1e-14, atol=1e-14), (b, h, np.abs(got - want).max())
        # write-back is the fp32 rounding of S'
        assert np.array_equal(pool[p.idx], r["state"].astype(np.float32))


def pin_output_gemv(o):
    p = _small(H=4, P=8, N=32, bs=3, slots=5, seed=31)
    _, r = _run(o, p)
    for b in range(p.batch):
        for h in range(p.nheads):
            S = r["state"][b, h]
            Cv = si.bf16_values(p.C[b, 0]).astype(np.float64)
            x = si.bf16_values(p.x[b, h]).astype(np.float64)
            terms = S * Cv[None, :]
            want = S @ Cv + np.float64(p.D[h]) * x
            tau = np.abs(terms).sum(axis=1) + np.abs(np.float64(p.D[h]) * x)
            assert np.all(np.abs(r["y"][b, h] - want) <= 1e-13 * tau), (b, h)
            assert np.allclose(r["tau"][b, h], tau, rtol=1e-13)
    import torch

    y32 = torch.from_numpy(r["y"].astype(np.float32))
    assert np.array_equal(r["out"], y32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def pin_gather(o):
    p = _small(H=2, P=8, N=16, bs=4, slots=11, seed=41)
    before = p.pool.copy()
    pool, r = _run(o, p)
    untouched = np.setdiff1d(np.arange(p.pool_slots), p.idx)
    assert np.array_equal(pool[untouched].view(np.uint32), before[untouched].view(np.uint32))
    assert not np.array_equal(pool[p.idx], before[p.idx])
    # permuting the requests (idx, x, B, C, dt together) permutes the outputs
    perm = np.array([2, 0, 3, 1])
    q = si.make_problem(2, 8, 16, 1, 4, 11, 41, idx=p.idx[perm])
    q.xbc = p.xbc[perm].copy()
    q.dt = p.dt[perm].copy()
    q.pool = before.copy()
    pool2, r2 = _run(o, q)
    assert np.array_equal(r2["out"], r["out"][perm])
    assert np.array_equal(pool2.view(np.uint32), pool.view(np.uint32))
    # slot ids outside [0, pool_slots) are padding: state and out rows untouched
    q.idx = np.array([p.idx[2], -1, p.idx[3], p.pool_slots], dtype=np.int32)
    q.xbc, q.dt = p.xbc.copy(), p.dt.copy()
    pool3 = before.copy()
    sentinel = np.full((4, 2, 8), 0x7FC1, dtype=np.uint16)
    r3 = o.run(pool3, q.idx, q.x, q.B, q.C, q.dt, q.A, q.dt_bias, q.D, out=sentinel)
    assert np.all(r3["out"][1] == 0x7FC1) and np.all(r3["out"][3] == 0x7FC1)
    assert not np.any(r3["out"][[0, 2]] == 0x7FC1)
    keep = np.setdiff1d(np.arange(p.pool_slots), q.idx[[0, 2]])
    assert np.array_equal(pool3[keep].view(np.uint32), before[keep].view(np.uint32))
    # duplicates are rejected
    q.idx = np.array([1, 2, 1, 3], dtype=np.int32)
    try:
        o.run(before.copy(), q.idx, q.x, q.B, q.C, q.dt, q.A, q.dt_bias, q.D)
    except ValueError as e:
        assert "duplicate" in str(e)
    else:
        raise AssertionError("duplicate slot ids accepted")


def pin_dt_zero(o):
    p = _small(H=3, P=8, N=16, bs=3, slots=6, seed=51, softplus=False)
    p.dt[:] = 0
    before = p.pool.copy()
    pool, r = _run(o, p, dt_bias=np.zeros(p.nheads, dtype=np.float32))
    assert np.array_equal(pool.view(np.uint32), before.view(np.uint32))
    for b in range(p.batch):
        for h in range(p.nheads):
            S0 = before[p.idx[b], h].astype(np.float64)
            Cv = si.bf16_values(p.C[b, 0]).astype(np.float64)
            x = si.bf16_values(p.x[b, h]).astype(np.float64)
            want = S0 @ Cv + np.float64(p.D[h]) * x
            tau = np.abs(S0 * Cv).sum(1) + np.abs(np.float64(p.D[h]) * x)
            assert np.all(np.abs(r["y"][b, h] - want) <= 1e-13 * tau)


def pin_A_very_negative(o):
    p = _small(H=3, P=8, N=16, bs=3, slots=6, seed=61)
    p.dt[:] = 0  # delta = softplus(dt_bias) in [1e-3, 0.1], so A*delta <= -1e6
    A = np.full(p.nheads, -1e9, dtype=np.float32)
    pool, r = _run(o, p, A=A)
    delta = np.logaddexp(0.0, p.dt_bias.astype(np.float64))
    for b in range(p.batch):
        for h in range(p.nheads):
            x = si.bf16_values(p.x[b, h]).astype(np.float64)
            Bv = si.bf16_values(p.B[b, 0]).astype(np.float64)
            Cv = si.bf16_values(p.C[b, 0]).astype(np.float64)
            want_state = np.outer(delta[h] * x, Bv)
            assert np.array_equal(pool[p.idx[b], h], want_state.astype(np.float32))
            want_y = x * (delta[h] * (Bv @ Cv) + np.float64(p.D[h]))
            scale = np.abs(x) * (delta[h] * np.abs(Bv) @ np.abs(Cv) + abs(float(p.D[h])))
            assert np.all(np.abs(r["y"][b, h] - want_y) <= 1e-13 * scale + 1e-300)


def pin_B_zero(o):
    p = _small(H=3, P=8, N=16, bs=3, slots=6, seed=71)
    o_ = p.nheads * p.headdim
    p.xbc[:, o_ : o_ + p.dstate] = 0
    before = p.pool.copy()
    pool, _ = _run(o, p)
    delta = _np_delta(p.dt, p.dt_bias[None, :], True)
    for b in range(p.batch):
        for h in range(p.nheads):
            a = np.exp(np.float64(p.A[h]) * delta[b, h])
            want = (a * before[p.idx[b], h].astype(np.float64)).astype(np.float32)
            assert np.array_equal(pool[p.idx[b], h], want)


def pin_C_zero(o):
    import torch

    p = _small(H=3, P=8, N=16, bs=3, slots=6, seed=81)
    o_ = p.nheads * p.headdim + p.dstate
    p.xbc[:, o_ : o_ + p.dstate] = 0
    _, r = _run(o, p)
    dx = torch.from_numpy(p.D[None, :, None].astype(np.float64) * si.bf16_values(p.x).astype(np.float64))
    want = dx.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r["out"], want)


def pin_groups(o):
    H, G, P, N, bs = 4, 2, 4, 8, 2
    p = si.make_problem(H, P, N, G, bs, 4, 91)
    before = p.pool.copy()
    pool, r = _run(o, p)
    delta = _np_delta(p.dt, p.dt_bias[None, :], True)
    for b in range(bs):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(np.float64(p.A[h]) * delta[b, h])
            x = si.bf16_values(p.x[b, h]).astype(np.float64)
            Bv = si.bf16_values(p.B[b, g]).astype(np.float64)
            Cv = si.bf16_values(p.C[b, g]).astype(np.float64)
            S = a * before[p.idx[b], h].astype(np.float64) + delta[b, h] * np.outer(x, Bv)
            assert np.allclose(r["state"][b, h], S, rtol=1e-14, atol=1e-14), (b, h)
            want = S @ Cv + np.float64(p.D[h]) * x
            assert np.allclose(r["y"][b, h], want, rtol=1e-12, atol=1e-12), (b, h)


def _scan_inputs(K, seed, H=2, P=4, N=8, bs=2, slots=5):
    base = si.make_problem(H, P, N, 1, bs, slots, seed)
    steps = [si.make_problem(H, P, N, 1, bs, slots, seed * 100 + t + 1, idx=base.idx) for t in range(K)]
    x = np.stack([s.x for s in steps])
    B = np.stack([s.B for s in steps])
    C = np.stack([s.C for s in steps])
    dt = np.stack([s.dt for s in steps])
    return base, x, B, C, dt


def pin_kstep(o):
    for K in (1, 2, 7, 32):
        base, x, B, C, dt = _scan_inputs(K, seed=100 + K)
        H, P, N, bs = base.nheads, base.headdim, base.dstate, base.batch
        S0 = base.pool.copy()
        pool_scan = S0.copy()
        r = o.run(pool_scan, base.idx, x, B, C, dt, base.A, base.dt_bias, base.D)
        delta = np.logaddexp(0.0, si.bf16_values(dt).astype(np.float64) + base.dt_bias[None, None, :])
        for b in range(bs):
            for h in range(H):
                Ah = np.float64(base.A[h])
                tot = delta[:, b, h].sum()
                want = np.exp(Ah * tot) * S0[base.idx[b], h].astype(np.float64)
                for t in range(K):
                    later = delta[t + 1 :, b, h].sum()
                    xt = si.bf16_values(x[t, b, h]).astype(np.float64)
                    Bt = si.bf16_values(B[t, b, 0]).astype(np.float64)
                    want = want + np.exp(Ah * later) * delta[t, b, h] * np.outer(xt, Bt)
                got = r["state"][b, h]
                assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (K, b, h, np.abs(got - want).max())
                # y_t uses the state after token t (closed form at t)
                t = K - 1
                Ct = si.bf16_values(C[t, b, 0]).astype(np.float64)
                xt = si.bf16_values(x[t, b, h]).astype(np.float64)
                yw = want @ Ct + np.float64(base.D[h]) * xt
                assert np.allclose(r["y"][t, b, h], yw, rtol=1e-11, atol=1e-11)
        # K single steps with fp32 storage in between stay within rounding of the scan
        pool_steps = S0.copy()
        for t in range(K):
            o.run(pool_steps, base.idx, x[t], B[t], C[t], dt[t], base.A, base.dt_bias, base.D)
        ref = r["state"]
        got = pool_steps[base.idx].astype(np.float64)
        assert np.all(np.abs(got - ref) <= K * 2.0 ** -23 * (1.0 + np.abs(ref)))


def pin_brute_force(o):
    rng = _rng(7)
    cases = [dict(H=2, P=64, N=128, G=1, bs=4, slots=8, seed=0)]  # the tiny workload itself
    for i in range(8):
        H = int(rng.integers(1, 5))
        G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
        cases.append(dict(H=H, P=int(rng.integers(1, 9)), N=int(rng.integers(1, 17)), G=G,
                          bs=int(rng.integers(1, 5)), slots=int(rng.integers(5, 9)), seed=200 + i))
    for c in cases:
        for softplus in (True, False):
            p = si.make_problem(c["H"], c["P"], c["N"], c["G"], c["bs"], c["slots"], c["seed"],
                                dt_softplus=softplus)
            before = p.pool.copy()
            pool, r = _run(o, p)
            new, y, out = brute.step(before.tolist(), p.idx.tolist(), p.x.tolist(), p.B.tolist(),
                                     p.C.tolist(), p.dt.tolist(), p.A.tolist(), p.dt_bias.tolist(),
                                     p.D.tolist(), softplus)
            new = np.array(new)
            S = new[p.idx]
            assert np.all(np.abs(r["state"] - S) <= 1e-13 * (1 + np.abs(S))), c
            assert np.array_equal(pool, new.astype(np.float32)), c
            y = np.array(y)
            assert np.all(np.abs(r["y"] - y) <= 1e-13 * (r["tau"] + 1e-300)), c
            out = np.array(out, dtype=np.uint16)
            agree = out == r["out"]
            if not agree.all():
                # only where the two sums' last-bit difference crosses a rounding boundary
                dist = np.abs(out[~agree].astype(np.int64) - r["out"][~agree].astype(np.int64))
                assert np.all(dist == 1) and np.all(r["y"][~agree] != y[~agree]), c


PINS = [
    pin_softplus_closed_forms,
    pin_bf16_rounding,
    pin_rank1_update,
    pin_output_gemv,
    pin_gather,
    pin_dt_zero,
    pin_A_very_negative,
    pin_B_zero,
    pin_C_zero,
    pin_groups,
    pin_kstep,
    pin_brute_force,
]


def pin_copy_blocks(o):
    """Block copy against numpy fancy-index assignment, the skip and no-op
    rules, and the rejection of order-dependent requests."""
    rng = _rng(12)
    tensors = [rng.standard_normal((9, 4, 6)).astype(np.float32),
               rng.integers(0, 65535, size=(9, 3, 5), dtype=np.uint16),
               rng.standard_normal((9, 7)).astype(np.float64)]
    before = [t.copy() for t in tensors]
    src = np.array([0, 3, 5, 7], dtype=np.int32)
    dst = np.array([1, 2, 8, 7], dtype=np.int32)  # last pair: src == dst, a no-op
    o.copy_blocks(tensors, src, dst)
    for t, b in zip(tensors, before):
        want = b.copy()
        want[dst[:3]] = b[src[:3]]
        assert np.array_equal(t, want)
    # out-of-range ids skip the request
    tensors2 = [b.copy() for b in before]
    o.copy_blocks(tensors2, np.array([-1, 4], dtype=np.int32), np.array([6, 9], dtype=np.int32))
    for t, b in zip(tensors2, before):
        assert np.array_equal(t, b)
    # a destination that is also a source, or two equal destinations: rejected
    for s_, d_ in (([0, 1], [1, 2]), ([0, 3], [4, 4])):
        try:
            o.copy_blocks([b.copy() for b in before], np.array(s_, dtype=np.int32), np.array(d_, dtype=np.int32))
        except ValueError:
            pass
        else:
            raise AssertionError(f"order-dependent copy accepted: {s_} -> {d_}")
    # a strided tensor (blocks not adjacent): only the block bytes move
    big = rng.standard_normal((6, 2, 8)).astype(np.float32)
    view = big[:, 0]  # block stride 64 bytes, block 32 bytes
    ref = big.copy()
    o.copy_blocks([view], np.array([1], dtype=np.int32), np.array([4], dtype=np.int32))
    ref[4, 0] = ref[1, 0]
    assert np.array_equal(big, ref)


PINS.append(pin_copy_blocks)


# --------------------------------------------------------------------------- #
# Selective scan over a sequence (prefill)
# --------------------------------------------------------------------------- #
def _scan_problem(io="f16", seed=21, batch=2, dim=4, N=3, G=2, L=9, zero_state=False, softplus=True):
    return si.make_scan_problem(batch, dim, N, L, G, io=io, seed=seed, zero_state=zero_state,
                                delta_softplus=softplus)


def _scan_run(o, p, state=None, **kw):
    state = p.state.copy() if state is None else state
    args = dict(D=p.D, delta_bias=p.delta_bias, delta_softplus=p.delta_softplus, io=p.io)
    args.update(kw)
    r = o.scan(state, args.pop("u", p.u), args.pop("delta", p.delta),
               args.pop("A", p.A), args.pop("B", p.B), args.pop("C", p.C), **args)
    return state, r


def _io_round(y, io):
    """numpy's RNE of fp32(y) into the io format, as bit patterns."""
    f = np.asarray(y, dtype=np.float64).astype(np.float32)
    if io == "f16":
        return f.astype(np.float16).view(np.uint16)
    return np.array([brute._bf16_bits_of_f32(float(v)) for v in f.ravel()], dtype=np.uint16).reshape(f.shape)


def pin_f16_decode(o):
    """Every binary16 bit pattern decodes to numpy's float16 value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_value(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_f16_rounding(o):
    """fp32 -> binary16 RNE matches numpy's conversion: random values across the
    range, exact ties between neighbours (normal and subnormal), the overflow
    threshold, signed zero, infinity and NaN."""
    rng = _rng(31)
    mag = np.exp2(rng.uniform(-30, 17, size=4000))
    vals = [mag * rng.choice([-1.0, 1.0], size=mag.size)]
    h = rng.integers(1, 0x7BFF, size=1000, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals.append((lo + hi) / 2)                       # ties, exact in fp32
    vals.append(np.array([65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                          2.0 ** -14 - 2.0 ** -25, 0.0, -0.0, np.inf, -np.inf]))
    v = np.concatenate(vals).astype(np.float32)
    got = o.f16_rne(v)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]
    n = o.f16_rne(np.array([np.nan], dtype=np.float32))
    assert np.isnan(n.view(np.float16)[0])


def pin_scan_brute_force(o):
    """The scan against the explicit-sum brute force: fp16 and bf16, softplus on
    and off, with and without D and delta_bias, two groups."""
    for io in ("f16", "bf16"):
        for softplus, with_opt in ((True, True), (False, True), (True, False)):
            p = _scan_problem(io=io, seed=22 + softplus + 2 * with_opt, softplus=softplus)
            if not softplus:
                # keep the steps positive and small without the softplus
                p.delta = si.io_bits(np.abs(si.io_values(p.delta, io)) * 0.25, io)
                p.delta_bias = np.full(p.dim, 0.01, dtype=np.float32)
            D, bias = (p.D, p.delta_bias) if with_opt else (None, None)
            state, r = _scan_run(o, p, D=D, delta_bias=bias)
            h, y, tau = brute.scan(p.state.tolist(), p.u.tolist(), p.delta.tolist(), p.A.tolist(), p.B.tolist(),
                                   p.C.tolist(), None if D is None else D.tolist(),
                                   None if bias is None else bias.tolist(), softplus, io, want_tau=True)
            h, y, tau = np.array(h), np.array(y), np.array(tau)
            assert np.allclose(r["state"], h, rtol=1e-12, atol=1e-14), (io, softplus, with_opt)
            assert np.all(np.abs(r["y"] - y) <= 1e-12 * (tau + 1e-300)), (io, softplus, with_opt)
            # tau exactly (both ways): sum_n |C h| + |D u| of the brute force's terms
            assert np.all(np.abs(r["tau"] - tau) <= 1e-12 * tau + 1e-300), (io, softplus, with_opt)
            assert np.array_equal(state, h.astype(np.float32))
            assert np.array_equal(r["out"], _io_round(r["y"], io))


def pin_scan_closed_form(o):
    """Constant inputs: with the same step, input and B at every token, each
    state follows the geometric series h_t = a^(t+1) h0 + beta (1 - a^(t+1)) / (1 - a),
    a = exp(A Delta), beta = Delta u B, with a distinct decay per state."""
    L, N, dim = 40, 4, 3
    p = _scan_problem(batch=1, dim=dim, N=N, G=1, L=L, seed=25)
    io = p.io
    uval, dval = np.float32(0.75), np.float32(-0.5)
    p.u = np.full_like(p.u, si.io_bits([uval], io)[0])
    p.delta = np.full_like(p.delta, si.io_bits([dval], io)[0])
    Bv = np.array([1.0, -2.0, 0.5, 3.0], dtype=np.float32)
    p.B = np.broadcast_to(si.io_bits(Bv, io)[None, None, :, None], p.B.shape).copy()
    p.C = np.broadcast_to(si.io_bits(np.ones(N, np.float32), io)[None, None, :, None], p.C.shape).copy()
    state, r = _scan_run(o, p)
    t = np.arange(L, dtype=np.float64)
    for d in range(dim):
        delta = np.logaddexp(0.0, float(dval) + float(p.delta_bias[d]))
        a = np.exp(p.A[d].astype(np.float64) * delta)               # [N]
        beta = delta * float(uval) * Bv.astype(np.float64)
        pw = a[:, None] ** (t[None, :] + 1)                          # [N, L]
        h = pw * p.state[0, d].astype(np.float64)[:, None] + beta[:, None] * (1 - pw) / (1 - a[:, None])
        y = h.sum(axis=0) + float(p.D[d]) * float(uval)
        assert np.allclose(r["y"][0, d], y, rtol=1e-12, atol=1e-13), d
        assert np.allclose(r["state"][0, d], h[:, -1], rtol=1e-12, atol=1e-14), d


def pin_scan_no_decay(o):
    """A = 0: no decay, the state is the running sum of the inputs
    (numpy.cumsum), and y = C . h + D u (numpy.einsum)."""
    p = _scan_problem(seed=26, L=30)
    p.A = np.zeros_like(p.A)
    state, r = _scan_run(o, p)
    io = p.io
    delta = np.logaddexp(0.0, si.io_values(p.delta, io).astype(np.float64) + p.delta_bias[None, :, None])
    u = si.io_values(p.u, io).astype(np.float64)
    g = np.arange(p.dim) // (p.dim // p.ngroups)
    B = si.io_values(p.B, io).astype(np.float64)[:, g]                # [b, dim, N, L]
    C = si.io_values(p.C, io).astype(np.float64)[:, g]
    h = p.state.astype(np.float64)[..., None] + np.cumsum((delta * u)[:, :, None, :] * B, axis=-1)
    y = np.einsum("bdnl,bdnl->bdl", h, C) + p.D[None, :, None] * u
    assert np.allclose(r["state"], h[..., -1], rtol=1e-12, atol=1e-13)
    assert np.all(np.abs(r["y"] - y) <= 1e-12 * (r["tau"] + 1e-300))


def pin_scan_memoryless(o):
    """A -> -1e30 makes every decay exactly 0: the state is the last token's
    input Delta u B, and y_t = C_t . (Delta_t u_t B_t) + D u_t."""
    p = _scan_problem(seed=27, L=11)
    p.A = np.full_like(p.A, -1e30)
    state, r = _scan_run(o, p)
    io = p.io
    delta = np.logaddexp(0.0, si.io_values(p.delta, io).astype(np.float64) + p.delta_bias[None, :, None])
    u = si.io_values(p.u, io).astype(np.float64)
    g = np.arange(p.dim) // (p.dim // p.ngroups)
    B = si.io_values(p.B, io).astype(np.float64)[:, g]
    C = si.io_values(p.C, io).astype(np.float64)[:, g]
    beta = (delta * u)[:, :, None, :] * B
    y = np.einsum("bdnl,bdnl->bdl", beta, C) + p.D[None, :, None] * u
    assert np.allclose(r["state"], beta[..., -1], rtol=1e-14, atol=0)
    assert np.all(np.abs(r["y"] - y) <= 1e-13 * (r["tau"] + 1e-300))


def pin_scan_zero_step(o):
    """Softplus off, delta = 0 and no bias: every step is 0, the state is left
    exactly as it was and y = C . h0 + D u."""
    p = _scan_problem(seed=28, softplus=False)
    p.delta = np.zeros_like(p.delta)
    state, r = _scan_run(o, p, delta_bias=None)
    assert np.array_equal(state, p.state)
    io = p.io
    g = np.arange(p.dim) // (p.dim // p.ngroups)
    C = si.io_values(p.C, io).astype(np.float64)[:, g]
    y = np.einsum("bdn,bdnl->bdl", p.state.astype(np.float64), C) \
        + p.D[None, :, None] * si.io_values(p.u, io).astype(np.float64)
    assert np.allclose(r["y"], y, rtol=1e-13, atol=1e-13)


def pin_scan_split(o):
    """Two scans over consecutive pieces of a sequence, the first's fp32 state
    carried into the second, agree with one scan over the whole (up to that
    fp32 rounding, which the error scale bounds), and the sequence of length 0
    changes nothing."""
    p = _scan_problem(seed=29, L=24, zero_state=False)
    whole_state, whole = _scan_run(o, p)
    st = p.state.copy()
    parts = []
    for t0, t1 in ((0, 10), (10, 24)):
        q = si.ScanProblem(**{**p.__dict__, "u": p.u[..., t0:t1], "delta": p.delta[..., t0:t1],
                              "B": p.B[..., t0:t1], "C": p.C[..., t0:t1], "seqlen": t1 - t0})
        _, r = _scan_run(o, q, state=st)
        parts.append(r)
    y = np.concatenate([parts[0]["y"], parts[1]["y"]], axis=-1)
    eps = 2.0 ** -24
    assert np.all(np.abs(y - whole["y"]) <= eps * (whole["rho"] + whole["tau"]))
    assert np.all(np.abs(st - whole["state"]) <= eps * whole["err"] + eps * np.abs(whole["state"]))
    q = si.ScanProblem(**{**p.__dict__, "u": p.u[..., :0], "delta": p.delta[..., :0], "B": p.B[..., :0],
                          "C": p.C[..., :0], "seqlen": 0})
    st0 = p.state.copy()
    _scan_run(o, q, state=st0)
    assert np.array_equal(st0, p.state)


def _fp32_scan(p):
    """Sequential fp32 scan in numpy (steps, decays, products and sums rounded
    to fp32, as a GPU kernel computes them). Returns (h, y)."""
    f32 = np.float32
    io = p.io
    v = (si.io_values(p.delta, io) + p.delta_bias[None, :, None]).astype(f32)
    delta = (np.maximum(v, f32(0)) + np.log1p(np.exp(-np.abs(v)))).astype(f32)
    u = si.io_values(p.u, io)
    du = (delta * u).astype(f32)
    B = si.io_values(p.B, io)[:, 0]
    C = si.io_values(p.C, io)[:, 0]
    h = p.state.copy()
    y = np.zeros(p.u.shape, f32)
    for t in range(p.seqlen):
        a = np.exp((p.A[None] * delta[:, :, t, None]).astype(f32)).astype(f32)
        h = (h * a + (du[:, :, t, None] * B[:, None, :, t]).astype(f32)).astype(f32)
        y[..., t] = ((h * C[:, None, :, t]).astype(f32).sum(axis=-1, dtype=f32)
                     + p.D[None] * u[..., t]).astype(f32)
    return h, y


def pin_scan_error_scale(o):
    """The error scales bound what fp32 arithmetic actually does: an fp32
    sequential scan in numpy stays within 4 * 2^-24 * E of the fp64 state and
    within 2^-24 * (rho + N tau) of y, and E >= |h| everywhere. Two regimes:
    the input recipe (short memory, mixed signs), and a long memory (decay
    rates ~1e-4 over 3000 tokens) with inputs of one sign, where fp32 rounding
    errors pile up over the whole sequence."""
    eps = 2.0 ** -24
    p = _scan_problem(seed=30, batch=1, dim=6, N=8, G=1, L=300, zero_state=False)
    _, r = _scan_run(o, p)
    h, y = _fp32_scan(p)
    assert np.all(np.abs(h - r["state"]) <= 4 * eps * r["err"])
    assert np.all(np.abs(y - r["y"]) <= eps * (r["rho"] + p.dstate * r["tau"]))
    assert np.all(r["err"] >= np.abs(r["state"]))

    p = _scan_problem(seed=31, batch=1, dim=6, N=8, G=1, L=3000, zero_state=True)
    p.A = np.broadcast_to(-1e-4 * (np.arange(8, dtype=np.float32) + 1), p.A.shape).astype(np.float32)
    p.u = si.io_bits(np.abs(si.io_values(p.u, p.io)) + 0.5, p.io)
    p.B = si.io_bits(np.abs(si.io_values(p.B, p.io)) + 0.5, p.io)
    _, r = _scan_run(o, p)
    h, _ = _fp32_scan(p)
    assert np.all(np.abs(h - r["state"]) <= 4 * eps * r["err"])


def pin_scan_error_scale_closed_forms(o):
    """The error scales equal their definitions, in closed form, from above and
    below. With beta_t = Delta_t u_t B_t and a_t = exp(A Delta_t) per state:
    M_t = a_t M_{t-1} + |beta_t|, E_t = a_t E_{t-1} + (1 + |A Delta_t|) a_t
    M_{t-1} + M_t, M_{-1} = E_{-1} = |h_{-1}|, rho_t = sum_n |C_t| E_t,
    tau_t = sum_n |h_t C_t| + |D u_t|.

    * Constant inputs (a, beta, C the same at every token): M_s = k + (m0 - k)
      a^(s+1) with k = |beta| / (1 - a), m0 = |h_{-1}|, and summing the two
      geometric series in E gives
      E_t = a^(t+1) m0 + (1 + c a) k (1 - a^(t+1)) / (1 - a)
            + (1 + c) (m0 - k) (t + 1) a^(t+1),   c = 1 + |A Delta|.
      Signed B, C and h_{-1}, so every absolute value matters.
    * A = 0 with every input positive: no decay, M_t = h_t = h_{-1} +
      cumsum(beta), and E_t = m0 + sum_{s<=t} (M_{s-1} + M_s) (numpy.cumsum).
    * A -> -1e30 (memoryless): E_t = M_t = |beta_t|, so rho_t = sum_n |C_t|
      |beta_t| and tau_t = sum_n |beta_t C_t| + |D u_t|.
    Agreement to 1e-12 relative: an error scale inflated (or deflated) by any
    factor fails."""
    rel = 1e-12

    def close(got, want):
        return np.all(np.abs(got - want) <= rel * np.abs(want) + 1e-300)

    # constant inputs, geometric series
    L, N, dim = 40, 4, 3
    p = _scan_problem(batch=1, dim=dim, N=N, G=1, L=L, seed=32, zero_state=False)
    io = p.io
    uval, dval = np.float32(0.75), np.float32(-0.5)
    p.u = np.full_like(p.u, si.io_bits([uval], io)[0])
    p.delta = np.full_like(p.delta, si.io_bits([dval], io)[0])
    Bv = np.array([1.0, -2.0, 0.5, 3.0], dtype=np.float32)
    Cv = np.array([1.5, -2.0, 0.25, -3.0], dtype=np.float32)
    p.B = np.broadcast_to(si.io_bits(Bv, io)[None, None, :, None], p.B.shape).copy()
    p.C = np.broadcast_to(si.io_bits(Cv, io)[None, None, :, None], p.C.shape).copy()
    _, r = _scan_run(o, p)
    t = np.arange(L, dtype=np.float64)[None, :]                       # [1, L]
    Cd = Cv.astype(np.float64)[:, None]                               # [N, 1]
    for d in range(dim):
        delta = np.logaddexp(0.0, float(dval) + float(p.delta_bias[d]))
        A = p.A[d].astype(np.float64)[:, None]
        a = np.exp(A * delta)
        beta = delta * float(uval) * Bv.astype(np.float64)[:, None]
        h0 = p.state[0, d].astype(np.float64)[:, None]
        m0, k, c = np.abs(h0), np.abs(beta) / (1 - a), 1 + np.abs(A * delta)
        pw = a ** (t + 1)
        h = pw * h0 + beta * (1 - pw) / (1 - a)
        E = pw * m0 + (1 + c * a) * k * (1 - pw) / (1 - a) + (1 + c) * (m0 - k) * (t + 1) * pw
        Du = abs(float(p.D[d]) * float(uval))
        assert close(r["err"][0, d], E[:, -1]), ("E", d)
        assert close(r["rho"][0, d], (np.abs(Cd) * E).sum(axis=0)), ("rho", d)
        assert close(r["tau"][0, d], np.abs(h * Cd).sum(axis=0) + Du), ("tau", d)

    # A = 0, all inputs positive: cumulative sums
    p = _scan_problem(batch=2, dim=4, N=3, G=2, L=25, seed=33, zero_state=False)
    io = p.io
    p.A = np.zeros_like(p.A)
    p.state = np.abs(p.state)
    p.u = si.io_bits(np.abs(si.io_values(p.u, io)) + 0.25, io)
    p.B = si.io_bits(np.abs(si.io_values(p.B, io)) + 0.25, io)
    _, r = _scan_run(o, p)
    delta = np.logaddexp(0.0, si.io_values(p.delta, io).astype(np.float64) + p.delta_bias[None, :, None])
    u = si.io_values(p.u, io).astype(np.float64)
    g = np.arange(p.dim) // (p.dim // p.ngroups)
    B = si.io_values(p.B, io).astype(np.float64)[:, g]                # [b, dim, N, L]
    C = si.io_values(p.C, io).astype(np.float64)[:, g]
    h0 = p.state.astype(np.float64)[..., None]                        # [b, dim, N, 1]
    h = h0 + np.cumsum((delta * u)[:, :, None, :] * B, axis=-1)       # = M
    hprev = np.concatenate([h0, h[..., :-1]], axis=-1)
    E = h0 + np.cumsum(hprev + h, axis=-1)
    assert close(r["err"], E[..., -1]), "E (A = 0)"
    assert close(r["rho"], (np.abs(C) * E).sum(axis=2)), "rho (A = 0)"
    assert close(r["tau"], np.abs(h * C).sum(axis=2) + np.abs(p.D[None, :, None] * u)), "tau (A = 0)"

    # memoryless
    p = _scan_problem(batch=2, dim=4, N=3, G=2, L=13, seed=34, zero_state=False)
    io = p.io
    p.A = np.full_like(p.A, -1e30)
    _, r = _scan_run(o, p)
    delta = np.logaddexp(0.0, si.io_values(p.delta, io).astype(np.float64) + p.delta_bias[None, :, None])
    u = si.io_values(p.u, io).astype(np.float64)
    B = si.io_values(p.B, io).astype(np.float64)[:, g]
    C = si.io_values(p.C, io).astype(np.float64)[:, g]
    beta = (delta * u)[:, :, None, :] * B
    assert close(r["err"], np.abs(beta[..., -1])), "E (memoryless)"
    assert close(r["rho"], (np.abs(C) * np.abs(beta)).sum(axis=2)), "rho (memoryless)"
    assert close(r["tau"], np.abs(beta * C).sum(axis=2) + np.abs(p.D[None, :, None] * u)), "tau (memoryless)"


def pin_scan_infinite_step(o):
    """A step of -inf with softplus on has size softplus(-inf) = 0: decay 1,
    input 0, so the scan is exactly the scan of the sequence with that token
    deleted (final state and every other token's y, bitwise in fp64), and its
    own y is C . h + D u of the state before it. Softplus of -inf is 0 in the
    limit; a form such as u + log1p(exp(-u)) gives NaN there."""
    p = _scan_problem(seed=31, L=12, zero_state=False)
    t = 5
    p.delta[..., t] = 0xFC00  # -inf (fp16)
    state, r = _scan_run(o, p)
    keep = np.array([k for k in range(p.seqlen) if k != t])
    q = si.ScanProblem(**{**p.__dict__, "u": p.u[..., keep], "delta": p.delta[..., keep], "B": p.B[..., keep],
                          "C": p.C[..., keep], "seqlen": p.seqlen - 1})
    q_state, rq = _scan_run(o, q)
    assert np.array_equal(r["state"], rq["state"]) and np.array_equal(state, q_state)
    assert np.array_equal(r["y"][..., keep], rq["y"])
    before = p.__dict__.copy()
    pre = si.ScanProblem(**{**before, "u": p.u[..., :t], "delta": p.delta[..., :t], "B": p.B[..., :t],
                            "C": p.C[..., :t], "seqlen": t})
    _, rp = _scan_run(o, pre)
    g = np.arange(p.dim) // (p.dim // p.ngroups)
    C_t = si.io_values(p.C[..., t], p.io).astype(np.float64)[:, g]        # [batch, dim, N]
    u_t = si.io_values(p.u[..., t], p.io).astype(np.float64)
    y_t = np.einsum("bdn,bdn->bd", rp["state"], C_t) + p.D[None, :] * u_t
    assert np.allclose(r["y"][..., t], y_t, rtol=1e-13, atol=1e-13)


PINS.extend([pin_f16_decode, pin_f16_rounding, pin_scan_brute_force, pin_scan_closed_form, pin_scan_no_decay,
             pin_scan_memoryless, pin_scan_zero_step, pin_scan_split, pin_scan_error_scale, pin_scan_error_scale_closed_forms,
             pin_scan_infinite_step])
