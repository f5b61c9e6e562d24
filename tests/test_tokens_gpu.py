"""Several decode tokens per request in one launch (ssu_update_tokens).

The fused call must be bitwise identical to the same tokens applied by
successive one-token ssu_update calls (the per-token arithmetic is the same
and the state stays fp32 between tokens), in every launch configuration, and
within tolerance of the oracle's fp64 length-K scan.
"""
import numpy as np
import pytest

import ssu_inputs as si

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


class TokenProblem:
    """K tokens for `batch` requests: per-token xBC rows packed as
    [batch, K, row] (x, B, C are views with a token axis), dt [batch, K, H];
    per-head parameters and slots shared by all tokens."""

    def __init__(self, H, P, N, G, batch, slots, K, seed, softplus=True, host_pool=True):
        self.base = si.make_problem(H, P, N, G, batch, slots, seed, dt_softplus=softplus, host_pool=host_pool)
        self.steps = []
        for t in range(K):
            s = si.make_problem(H, P, N, G, batch, slots, seed * 100 + t + 1, dt_softplus=softplus,
                                host_pool=False, idx=self.base.idx)
            s.A, s.D, s.dt_bias = self.base.A, self.base.D, self.base.dt_bias
            self.steps.append(s)
        self.H, self.P, self.N, self.G, self.bs, self.K = H, P, N, G, batch, K
        self.xbc = np.stack([s.xbc for s in self.steps], axis=1)  # [bs, K, row]
        self.dt = np.stack([s.dt for s in self.steps], axis=1)    # [bs, K, H]

    def device(self, pool):
        torch = gu.torch_mod()
        H, P, N, G, bs, K = self.H, self.P, self.N, self.G, self.bs, self.K
        xbc = gu.bf16_tensor(self.xbc, "cuda")
        row = xbc.shape[2]
        d = dict(
            pool=pool, xbc=xbc,
            x=xbc.as_strided((bs, K, H, P), (K * row, row, P, 1), 0),
            B=xbc.as_strided((bs, K, G, N), (K * row, row, N, 1), H * P),
            C=xbc.as_strided((bs, K, G, N), (K * row, row, N, 1), H * P + G * N),
            dt=gu.bf16_tensor(self.dt, "cuda"),
            A=torch.from_numpy(self.base.A).cuda(), D=torch.from_numpy(self.base.D).cuda(),
            dt_bias=torch.from_numpy(self.base.dt_bias).cuda(), idx=torch.from_numpy(self.base.idx).cuda())
        return d

    def oracle(self, ref, pool_np, sample=None):
        b = slice(None) if sample is None else sample
        x = np.stack([s.x[b] for s in self.steps])
        B = np.stack([s.B[b] for s in self.steps])
        C = np.stack([s.C[b] for s in self.steps])
        dt = np.stack([s.dt[b] for s in self.steps])
        idx = self.base.idx if sample is None else np.arange(len(sample), dtype=np.int32)
        return ref.run(pool_np, idx, x, B, C, dt, self.base.A, self.base.dt_bias, self.base.D,
                       self.base.dt_softplus)


def _fused_and_sequential(tp, h):
    torch = gu.torch_mod()
    pool0 = torch.from_numpy(tp.base.pool).cuda()
    d = tp.device(pool0.clone())
    out_f = h.update_tokens(d["pool"], d["idx"], d["x"], d["B"], d["C"], d["dt"], d["A"], d["D"], d["dt_bias"])
    pool_seq = pool0.clone()
    outs = []
    for t in range(tp.K):
        outs.append(h.update(pool_seq, d["idx"], d["x"][:, t], d["B"][:, t], d["C"][:, t], d["dt"][:, t],
                             d["A"], d["D"], d["dt_bias"]))
    torch.cuda.synchronize()
    return d["pool"], out_f, pool_seq, torch.stack(outs, dim=1)


@pytest.mark.parametrize("N,P,H,G,bs,K", [
    (128, 64, 4, 1, 6, 1), (128, 64, 4, 1, 6, 2), (128, 64, 4, 1, 6, 3), (128, 64, 4, 1, 5, 8),
    (64, 32, 4, 2, 5, 3), (256, 64, 2, 1, 4, 4), (16, 64, 4, 1, 3, 5), (32, 128, 2, 2, 3, 2),
])
def test_tokens_match_sequential_bitwise_and_oracle(ref, N, P, H, G, bs, K):
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    tp = TokenProblem(H, P, N, G, bs, 2 * bs + 1, K, seed=3000 + N + P + K)
    h = ssu.Handle(H, P, N, G, True)
    pool_f, out_f, pool_s, out_s = _fused_and_sequential(tp, h)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16)), "out differs from sequential"
    assert torch.equal(pool_f.view(torch.int32), pool_s.view(torch.int32)), "state differs from sequential"
    pool_ref = tp.base.pool.copy()
    r = tp.oracle(ref, pool_ref)
    gpu = pool_f.cpu().numpy()
    gu.assert_state(gpu[tp.base.idx], r["state"], f"K={K} state")
    ob = gu.bits(out_f)  # [bs, K, H, P]
    for t in range(K):
        gu.assert_out(ob[:, t], {k: r[k][t] for k in ("out", "y", "tau")}, f"K={K} token {t}")
    untouched = np.setdiff1d(np.arange(tp.base.pool_slots), tp.base.idx)
    assert np.array_equal(gpu[untouched].view(np.uint32), tp.base.pool[untouched].view(np.uint32))


@pytest.mark.parametrize("N", [128, 16, 32, 64, 256])
def test_tokens_every_tile_bitwise(ref, N):
    """Every launch configuration of every dstate (each splits a state row
    over its own number of lanes and sums rows in its own grouping) gives the
    same bits; the first is also checked against the oracle."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    tp = TokenProblem(4, 64, N, 1, 6, 13, 3, seed=3100 + N)
    base = None
    ids = [x for x in ssu.tiles() if x["dstate"] == N and ssu.tile_fits(x, 4, 64)]
    assert ids
    for t in ids:
        h = ssu.Handle(4, 64, N, 1, True, t["id"])
        pool = torch.from_numpy(tp.base.pool).cuda()
        d = tp.device(pool)
        o = h.update_tokens(d["pool"], d["idx"], d["x"], d["B"], d["C"], d["dt"], d["A"], d["D"], d["dt_bias"])
        torch.cuda.synchronize()
        if base is None:
            base = (o.clone(), pool.clone())
            r = tp.oracle(ref, tp.base.pool.copy())
            gu.assert_state(pool.cpu().numpy()[tp.base.idx], r["state"], f"N={N} {t['name']} state")
            ob = gu.bits(o)
            for k in range(tp.K):
                gu.assert_out(ob[:, k], {key: r[key][k] for key in ("out", "y", "tau")}, f"N={N} token {k}")
        else:
            assert torch.equal(o.view(torch.int16), base[0].view(torch.int16)), t["name"]
            assert torch.equal(pool.view(torch.int32), base[1].view(torch.int32)), t["name"]


def test_tokens_padding():
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    tp = TokenProblem(4, 64, 128, 1, 5, 11, 4, seed=3200)
    tp.base.idx[2] = -1
    h = ssu.Handle(4, 64, 128, 1, True)
    pool = torch.from_numpy(tp.base.pool).cuda()
    d = tp.device(pool)
    out = torch.full((5, 4, 4, 64), 0.25, dtype=torch.bfloat16, device="cuda")
    h.update_tokens(d["pool"], d["idx"], d["x"], d["B"], d["C"], d["dt"], d["A"], d["D"], d["dt_bias"], out)
    torch.cuda.synchronize()
    assert torch.all(out[2] == 0.25)
    live = tp.base.idx[tp.base.idx >= 0]
    untouched = np.setdiff1d(np.arange(11), live)
    assert np.array_equal(pool.cpu().numpy()[untouched], tp.base.pool[untouched])


@pytest.mark.parametrize("K,tile", [(2, "n128_r8_w1_nt_xcd_g14"), (3, "n128_r8_w1_nt_xcd_g20"),
                                    (4, "n128_r8_w1_nt_xcd"), (8, "n128_r16_w1_nt_xcd"),
                                    (16, "n128_r16_w2_nt_xcd")])
def test_tokens_headline_shape(ref, K, tile):
    """H16 P64 N128, batch 512, K tokens (the state read and written once), in
    the launch configuration the library picks for K: every request against
    the oracle's scan."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    bs = 512
    tp = TokenProblem(16, 64, 128, 1, bs, bs, K, seed=3300 + K, host_pool=False)
    pool = torch.empty((bs, 16, 64, 128), device="cuda")
    si.draw_pool_on_device(pool, 3300)
    before = pool.clone()
    h = ssu.Handle(16, 64, 128, 1, True)
    assert ssu.tiles()[h.selected_tile(bs, K)]["name"] == tile
    d = tp.device(pool)
    out = h.update_tokens(d["pool"], d["idx"], d["x"], d["B"], d["C"], d["dt"], d["A"], d["D"], d["dt_bias"])
    torch.cuda.synchronize()
    sample = np.arange(bs)
    sl = torch.from_numpy(tp.base.idx[sample].astype(np.int64)).cuda()
    r = tp.oracle(ref, before[sl].cpu().numpy(), sample=sample)
    gu.assert_state(pool[sl].cpu().numpy(), r["state"], "tokens headline")
    ob = gu.bits(out)[sample]
    for t in range(K):
        gu.assert_out(ob[:, t], {k: r[k][t] for k in ("out", "y", "tau")}, f"tokens headline t{t}")


def test_tokens_hip_graph_replays_match_eager(ref):
    """Two 3-token calls on disjoint slot sets captured in one HIP graph and
    replayed three times with eager work in between: every replay equals the
    eager round from the same state, and the first round matches the oracle."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    K = 3
    tp = TokenProblem(4, 64, 128, 1, 5, 10, K, seed=3400)
    other = np.setdiff1d(np.arange(10), tp.base.idx).astype(np.int32)
    idx_sets = [torch.from_numpy(tp.base.idx).cuda(), torch.from_numpy(other).cuda()]
    h = ssu.Handle(4, 64, 128, 1, True)
    pool = torch.from_numpy(tp.base.pool).cuda()
    d = tp.device(pool)
    outs = [torch.empty((5, K, 4, 64), dtype=torch.bfloat16, device="cuda") for _ in idx_sets]

    def calls():
        for i, o in zip(idx_sets, outs):
            h.update_tokens(pool, i, d["x"], d["B"], d["C"], d["dt"], d["A"], d["D"], d["dt_bias"], o)

    start = pool.clone()
    eager = []
    for _ in range(3):
        calls()
        torch.cuda.synchronize()
        eager.append((pool.clone(), [o.clone() for o in outs]))
    pool.copy_(start)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    pool.copy_(start)
    torch.cuda.synchronize()
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = (pool[:1].sum() + 1).item()  # eager work between replays
        want_pool, want_outs = eager[k]
        assert torch.equal(pool.view(torch.int32), want_pool.view(torch.int32)), f"replay {k} state"
        for o, w in zip(outs, want_outs):
            assert torch.equal(o.view(torch.int16), w.view(torch.int16)), f"replay {k} out"
    r = tp.oracle(ref, tp.base.pool.copy())
    gu.assert_state(eager[0][0].cpu().numpy()[tp.base.idx], r["state"], "graph round 0")


@pytest.mark.parametrize("K", [100, 1024])
def test_tokens_beyond_one_discretisation_batch(ref, K):
    """More tokens than one wave discretises at once (64 per batch, one per
    lane), up to the maximum of 1024: the fused call still equals K successive
    one-token calls bitwise, and the oracle's fp64 scan within the state and
    out tolerances (the decays keep fp32 rounding from accumulating: an fp32
    emulation stays near 1e-7 relative at K = 1024)."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    tp = TokenProblem(2, 64, 128, 1, 3, 7, K, seed=3500 + K)
    h = ssu.Handle(2, 64, 128, 1, True)
    pool_f, out_f, pool_s, out_s = _fused_and_sequential(tp, h)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16)), "out differs from sequential"
    assert torch.equal(pool_f.view(torch.int32), pool_s.view(torch.int32)), "state differs from sequential"
    r = tp.oracle(ref, tp.base.pool.copy())
    gu.assert_state(pool_f.cpu().numpy()[tp.base.idx], r["state"], f"K={K} state")
    ob = gu.bits(out_f)
    for t in (0, 63, 64, K - 1):
        gu.assert_out(ob[:, t], {k: r[k][t] for k in ("out", "y", "tau")}, f"K={K} token {t}")


@pytest.mark.parametrize("case", range(8))
def test_tokens_random_shapes(ref, case):
    """Seeded random K-token calls: d_state, headdim, heads, groups, batch and
    K (1 .. 80) drawn together; fused = sequential bitwise, and the oracle's
    fp64 scan within tolerance."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    rng = np.random.Generator(np.random.PCG64([89, case]))
    N = int(rng.choice([16, 32, 64, 128, 256]))
    P = 16 * int(rng.integers(1, 17))
    H = int(rng.integers(1, 9))
    G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
    bs = int(rng.integers(1, 9))
    K = int(rng.integers(1, 81))
    print(f"case {case}: N {N} P {P} H {H} G {G} bs {bs} K {K}", flush=True)
    tp = TokenProblem(H, P, N, G, bs, bs + 3, K, seed=3600 + case)
    h = ssu.Handle(H, P, N, G, True)
    pool_f, out_f, pool_s, out_s = _fused_and_sequential(tp, h)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16)), "out differs from sequential"
    assert torch.equal(pool_f.view(torch.int32), pool_s.view(torch.int32)), "state differs from sequential"
    r = tp.oracle(ref, tp.base.pool.copy())
    gu.assert_state(pool_f.cpu().numpy()[tp.base.idx], r["state"], f"case {case} state")
    ob = gu.bits(out_f)
    for t in sorted({0, K // 2, K - 1}):
        gu.assert_out(ob[:, t], {k: r[k][t] for k in ("out", "y", "tau")}, f"case {case} token {t}")
