"""libssu on the GPU against the CPU oracle, element by element.

Every test calls the HIP kernel through the C ABI (the Python binding only
marshals arguments) and compares with oracle/ on the same seeded inputs:
state within 1e-5 * (1 + |ref|), out within 2 bf16 ulp of bf16(fp32(y)) (with
the cancellation floor of tests/tolerance.py), untouched slots bitwise
unchanged, reruns and launch configurations bitwise identical.
"""
import ctypes

import numpy as np
import pytest

import ssu_inputs as si

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _problem(cfg_id, pool_slots=None):
    c = dict(si.CONFIGS[cfg_id])
    c.pop("name")
    if pool_slots is not None:
        c["pool_slots"] = pool_slots
    elif "pool_slots" not in c:
        c["pool_slots"] = 2 * c["batch"]
    return si.make_problem(**c)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_config_parity_and_rerun(ref, cfg):
    torch = gu.torch_mod()
    p = _problem(cfg)
    print(f"config {cfg}: {si.CONFIGS[cfg]['name']}", flush=True)
    dp = gu.DeviceProblem(p)
    pool0 = p.pool.copy()
    backup = dp.pool.clone()
    h = dp.handle()
    out = dp.run(h)
    torch.cuda.synchronize()
    _, pool_gpu, out_bits, floor = gu.compare_full(ref, dp, pool0, out, f"config {cfg}")
    print(f"config {cfg}: tile {h.selected_tile(p.batch)}, floor passes {floor}", flush=True)
    # rerun from the restored pool: bitwise equal
    dp.pool.copy_(backup)
    out2 = dp.run(h, out=torch.empty_like(out))
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits(out2), out_bits)
    assert np.array_equal(dp.pool.cpu().numpy().view(np.uint32), pool_gpu.view(np.uint32))


@pytest.mark.parametrize("N,P", [(128, 64), (16, 64), (32, 64), (64, 64), (256, 64), (128, 32)])
def test_every_tile_bitwise_identical(ref, N, P):
    """All launch configurations give the same bits (fixed reduction order)."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=P, N=N, G=1, batch=6, pool_slots=13, seed=500 + N + P)
    dp = gu.DeviceProblem(p)
    backup = dp.pool.clone()
    base_out = dp.run(tile=-1).clone()
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), base_out, f"N{N} P{P} auto")
    base_pool = dp.pool.clone()
    ids = [t["id"] for t in ssu.tiles() if t["dstate"] == N and ssu.tile_fits(t, 4, P)]
    assert ids
    for tid in ids:
        dp.pool.copy_(backup)
        o = dp.run(tile=tid, out=torch.empty_like(base_out))
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), base_out.view(torch.int16)), f"tile {tid} out differs"
        assert torch.equal(dp.pool.view(torch.int32), base_pool.view(torch.int32)), f"tile {tid} state differs"


@pytest.mark.parametrize("N", [16, 32])
def test_multihead_tiles_bitwise_identical(ref, N):
    """Groups whose waves each take a whole head of one request (2 to 16 heads
    per group at H = 16, P = 64) give the same bits as the library's choice,
    which matches the oracle; padding entries skip all of a group's heads."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    H, P = 16, 64
    p = si.make_problem(H=H, P=P, N=N, G=2, batch=5, pool_slots=11, seed=530 + N)
    idx = p.idx.copy()
    idx[3] = -1
    p.idx = idx
    dp = gu.DeviceProblem(p)
    backup = dp.pool.clone()
    base_out = dp.run(tile=-1).clone()
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), base_out, f"N{N} multi-head auto")
    base_pool = dp.pool.clone()
    ids = [t["id"] for t in ssu.tiles() if t["dstate"] == N and ssu.tile_fits(t, H, P) and t["rows_per_group"] > P]
    assert len(ids) >= 4
    for tid in ids:
        dp.pool.copy_(backup)
        o = dp.run(tile=tid, out=base_out.clone())
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), base_out.view(torch.int16)), f"tile {tid} out differs"
        assert torch.equal(dp.pool.view(torch.int32), base_pool.view(torch.int32)), f"tile {tid} state differs"


@pytest.mark.parametrize("N,P,H,G,bs", [
    (16, 64, 4, 1, 5), (32, 32, 4, 2, 7), (64, 64, 8, 4, 3), (256, 64, 4, 1, 9), (128, 16, 6, 3, 4),
    (128, 128, 4, 1, 6), (128, 256, 2, 2, 3), (64, 80, 4, 1, 5), (128, 64, 8, 8, 4), (256, 256, 2, 1, 3),
])
def test_shapes_groups_parity(ref, N, P, H, G, bs):
    torch = gu.torch_mod()
    p = si.make_problem(H=H, P=P, N=N, G=G, batch=bs, pool_slots=2 * bs + 1, seed=600 + N + P + H + G)
    dp = gu.DeviceProblem(p)
    out = dp.run()
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), out, f"N{N} P{P} H{H} G{G} bs{bs}")


@pytest.mark.parametrize("softplus,use_bias,use_D", [(False, True, True), (True, False, True),
                                                     (True, True, False), (False, False, False)])
def test_options_parity(ref, softplus, use_bias, use_D):
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=8, pool_slots=17, seed=700, dt_softplus=softplus)
    dp = gu.DeviceProblem(p)
    out = dp.run(use_bias=use_bias, use_D=use_D)
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), out, f"softplus={softplus} bias={use_bias} D={use_D}",
                    use_bias=use_bias, use_D=use_D)


def test_padding_and_int64_indices(ref):
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=6, pool_slots=10, seed=800)
    idx = p.idx.copy()
    idx[1] = -1
    idx[4] = p.pool_slots  # one past the end: padding too
    p.idx = idx
    dp = gu.DeviceProblem(p)
    sentinel = torch.full((6, 4, 64), 0.5, dtype=torch.bfloat16, device="cuda")
    out = dp.run(out=sentinel)
    torch.cuda.synchronize()
    r, pool_gpu, out_bits, _ = gu.compare_full(ref, dp, p.pool.copy(), out, "padding")
    half = gu.bits(torch.tensor([0.5], dtype=torch.bfloat16))[0]
    assert np.all(out_bits[[1, 4]] == half), "padding rows written"
    # int64 indices: bitwise the same as int32
    dp2 = gu.DeviceProblem(p)
    o64 = dp2.run(idx=dp2.idx.to(torch.int64), out=torch.full_like(sentinel, 0.5))
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits(o64), out_bits)
    assert np.array_equal(dp2.pool.cpu().numpy().view(np.uint32), pool_gpu.view(np.uint32))


@pytest.mark.parametrize("offset", [0, 1], ids=["first_low_half", "first_high_half"])
def test_dt_at_the_edges_of_its_allocation(ref, offset):
    """dt is read as the aligned words that hold its elements. A dt view that
    fills its own allocation exactly, with an odd element count (batch 5 x 3
    heads), has its last element in the low half of a word when it starts on a
    word (offset 0) and its first element in the high half of a word when it
    starts 2 bytes in (offset 1): the results match the oracle either way, for
    the one-token and the K-token call."""
    torch = gu.torch_mod()
    p = si.make_problem(H=3, P=64, N=128, batch=5, pool_slots=11, seed=810)
    dp = gu.DeviceProblem(p)
    storage = torch.empty(p.batch * p.nheads + offset, dtype=torch.bfloat16, device="cuda")
    storage[offset:] = gu.bf16_tensor(p.dt.ravel(), "cuda")
    dt = storage[offset:].view(p.batch, p.nheads)
    assert dt.data_ptr() % 4 == 2 * offset
    h = dp.handle()
    out = torch.empty_like(dp.out)
    h.update(dp.pool, dp.idx, dp.x, dp.B, dp.C, dt, dp.A, dp.D, dp.dt_bias, out)
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), out, f"dt offset {offset}")
    # a 3-token call whose dt [batch, 3, H] fills its allocation the same way
    # equals three one-token calls bitwise
    K = 3
    dts = np.random.Generator(np.random.PCG64(811)).standard_normal((p.batch, K, p.nheads)).astype(np.float32)
    storage = torch.empty(p.batch * K * p.nheads + offset, dtype=torch.bfloat16, device="cuda")
    storage[offset:] = torch.from_numpy(dts.ravel()).to(torch.bfloat16).cuda()
    dtk = storage[offset:].view(p.batch, K, p.nheads)
    xk, Bk, Ck = (v[:, None].expand(v.shape[0], K, *v.shape[1:]) for v in (dp.x, dp.B, dp.C))
    pool_k = torch.from_numpy(p.pool).cuda()
    out_k = h.update_tokens(pool_k, dp.idx, xk, Bk, Ck, dtk, dp.A, dp.D, dp.dt_bias)
    pool_s = torch.from_numpy(p.pool).cuda()
    for t in range(K):
        o = h.update(pool_s, dp.idx, dp.x, dp.B, dp.C, dtk[:, t], dp.A, dp.D, dp.dt_bias)
        torch.cuda.synchronize()
        assert torch.equal(out_k[:, t].view(torch.int16), o.view(torch.int16)), (offset, t)
    assert torch.equal(pool_k.view(torch.int32), pool_s.view(torch.int32)), offset


def test_request_permutation_bitwise(ref):
    """Requests are independent: permuting (idx, x, B, C, dt) together over
    the batch permutes out the same way, bitwise, and leaves the same pool,
    in launch configurations with and without XCD-ordered workgroups."""
    import dataclasses

    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=11, pool_slots=25, seed=810)
    perm = np.random.default_rng(810).permutation(p.batch)
    q = dataclasses.replace(p, xbc=p.xbc[perm].copy(), dt=p.dt[perm].copy(), idx=p.idx[perm].copy())
    tiles = [-1] + [t["id"] for t in ssu.tiles()
                    if t["name"] in ("n128_r8_w1_nt_xcd_g12", "n128_r4_w2_nt", "n128_r16_w2_xcd")]
    assert len(tiles) == 4
    for tile in tiles:
        dp, dq = gu.DeviceProblem(p), gu.DeviceProblem(q)
        op = dp.run(tile=tile)
        oq = dq.run(tile=tile)
        torch.cuda.synchronize()
        if tile == -1:
            gu.compare_full(ref, dp, p.pool.copy(), op, "unpermuted")
        assert np.array_equal(gu.bits(oq), gu.bits(op)[perm]), f"tile {tile}: out not permuted alike"
        assert torch.equal(dq.pool.view(torch.int32), dp.pool.view(torch.int32)), f"tile {tile}: pools differ"


def test_dt_zero_leaves_state_unchanged(ref):
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=5, pool_slots=9, seed=900, dt_softplus=False)
    p.dt[:] = 0
    dp = gu.DeviceProblem(p)
    before = dp.pool.clone()
    out = dp.run(use_bias=False)
    torch.cuda.synchronize()
    assert torch.equal(dp.pool.view(torch.int32), before.view(torch.int32))
    gu.compare_full(ref, dp, p.pool.copy(), out, "dt=0", use_bias=False)


def test_C_zero_gives_D_x_exactly(ref):
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=5, pool_slots=9, seed=901)
    o = p.nheads * p.headdim + p.ngroups * p.dstate
    p.xbc[:, o:] = 0
    dp = gu.DeviceProblem(p)
    out = dp.run()
    torch.cuda.synchronize()
    want = (dp.D[None, :, None].double() * dp.x.double()).float().to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    gu.compare_full(ref, dp, p.pool.copy(), out, "C=0")


def test_very_negative_A_collapses_state(ref):
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=5, pool_slots=9, seed=902)
    p.dt[:] = 0
    p.A[:] = -1e9
    dp = gu.DeviceProblem(p)
    out = dp.run()
    torch.cuda.synchronize()
    r, pool_gpu, _, _ = gu.compare_full(ref, dp, p.pool.copy(), out, "A=-1e9")
    # closed form: S' = delta * x[p] * B[n]
    delta = np.logaddexp(0.0, p.dt_bias.astype(np.float64))
    xs = si.bf16_values(p.x).astype(np.float64)
    Bs = si.bf16_values(p.B[:, 0]).astype(np.float64)
    want = delta[None, :, None, None] * xs[:, :, :, None] * Bs[:, None, None, :]
    gu.assert_state(pool_gpu[p.idx], want, "closed form")


@pytest.mark.parametrize("K", [2, 7, 32])
def test_k_successive_steps_match_scan(ref, K):
    """K decode calls equal the oracle's sequential length-K scan."""
    torch = gu.torch_mod()
    base = si.make_problem(H=4, P=64, N=128, batch=6, pool_slots=11, seed=1000 + K)
    steps = [si.make_problem(H=4, P=64, N=128, batch=6, pool_slots=11, seed=2000 + 10 * K + t, idx=base.idx)
             for t in range(K)]
    for s in steps:  # the per-head parameters are the layer's weights: the same for every token
        s.A, s.D, s.dt_bias = base.A, base.D, base.dt_bias
    dev = gu.DeviceProblem(base)
    h = dev.handle()
    outs = []
    for s in steps:
        d = gu.DeviceProblem(s, pool=dev.pool)
        outs.append(d.run(h).clone())
    torch.cuda.synchronize()
    x = np.stack([s.x for s in steps])
    B = np.stack([s.B for s in steps])
    C = np.stack([s.C for s in steps])
    dt = np.stack([s.dt for s in steps])
    pool_ref = base.pool.copy()
    r = ref.run(pool_ref, base.idx, x, B, C, dt, base.A, base.dt_bias, base.D)
    gpu = dev.pool.cpu().numpy()
    gu.assert_state(gpu[base.idx], r["state"], f"K={K} state")
    for t in (0, K - 1):
        gu.assert_out(gu.bits(outs[t]), {k: r[k][t] for k in ("out", "y", "tau")}, f"K={K} out[{t}]")


def test_hip_graph_replays_match_eager(ref):
    """Three updates captured in one HIP graph, replayed three times with eager
    work in between; every replay equals the eager run from the same state."""
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=6, pool_slots=24, seed=1100)
    sets = [np.arange(6, dtype=np.int32) + 6 * k for k in range(3)]
    dp = gu.DeviceProblem(p)
    h = dp.handle()
    idxs = [torch.from_numpy(s).cuda() for s in sets]
    outs = [torch.empty_like(dp.out) for _ in sets]

    def calls():
        for i, o in zip(idxs, outs):
            h.update(dp.pool, i, dp.x, dp.B, dp.C, dp.dt, dp.A, dp.D, dp.dt_bias, o)

    start = dp.pool.clone()
    # eager reference of three successive rounds
    eager = []
    for _ in range(3):
        calls()
        torch.cuda.synchronize()
        eager.append((dp.pool.clone(), [o.clone() for o in outs]))
    dp.pool.copy_(start)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        calls()  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    dp.pool.copy_(start)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    dp.pool.copy_(start)  # capture does not run the work
    torch.cuda.synchronize()
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = (dp.pool[:1].sum() + 1).item()  # eager work between replays
        want_pool, want_outs = eager[k]
        assert torch.equal(dp.pool.view(torch.int32), want_pool.view(torch.int32)), f"replay {k} state"
        for o, w in zip(outs, want_outs):
            assert torch.equal(o.view(torch.int16), w.view(torch.int16)), f"replay {k} out"
    # and the first round is right against the oracle
    pool_ref = p.pool.copy()
    for s_ in sets:
        r = ref.run(pool_ref, s_, p.x, p.B, p.C, p.dt, p.A, p.dt_bias, p.D)
    gu.assert_state(eager[0][0].cpu().numpy()[sets[2]], r["state"], "graph round 0, set 2")


def test_batch_zero_and_functional_api(ref):
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    p = si.make_problem(H=2, P=64, N=128, batch=4, pool_slots=8, seed=0)
    dp = gu.DeviceProblem(p)
    before = dp.pool.clone()
    empty = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    eB = torch.empty(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    o = ssu.selective_state_update(dp.pool, empty, torch.empty(0, 2, dtype=torch.bfloat16, device="cuda"),
                                   dp.A, eB, eB, dp.D, dp.dt_bias, True,
                                   torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64) and torch.equal(dp.pool, before)
    out = ssu.selective_state_update(dp.pool, dp.x, dp.dt, dp.A, dp.B, dp.C, dp.D, dp.dt_bias, True, dp.idx)
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), out, "functional")


def test_check_indices_detects_duplicates():
    import selective_state_update_amd as ssu

    p = si.make_problem(H=2, P=64, N=128, batch=4, pool_slots=8, seed=3)
    dp = gu.DeviceProblem(p)
    h = dp.handle()
    h.update(dp.pool, dp.idx, dp.x, dp.B, dp.C, dp.dt, dp.A, dp.D, dp.dt_bias, dp.out, check_indices=True)
    dup = dp.idx.clone()
    dup[3] = dup[0]
    with pytest.raises(ssu.SSUError, match=r"BAD_INDEX.*idx\[3\].*repeats idx\[0\]"):
        h.update(dp.pool, dup, dp.x, dp.B, dp.C, dp.dt, dp.A, dp.D, dp.dt_bias, dp.out, check_indices=True)

    # padding entries (outside [0, pool_slots)) may repeat
    pad = dp.idx.clone()
    pad[1], pad[2] = -1, 8
    pad[3] = -1
    args = h.make_args(dp.pool, pad, dp.x, dp.B, dp.C, dp.dt, dp.A, dp.D, dp.dt_bias, dp.out)
    assert ssu._lib.ssu_check_indices(ctypes.byref(args), None) == 0

    # the check needs no memory in proportion to the pool: a pool of 2^40
    # slots (never dereferenced here) is checked like any other
    args = h.make_args(dp.pool, dup, dp.x, dp.B, dp.C, dp.dt, dp.A, dp.D, dp.dt_bias, dp.out)
    args.pool_slots = 1 << 40
    assert ssu._lib.ssu_check_indices(ctypes.byref(args), None) == 6
    args = h.make_args(dp.pool, dp.idx, dp.x, dp.B, dp.C, dp.dt, dp.A, dp.D, dp.dt_bias, dp.out)
    args.pool_slots = 1 << 40
    assert ssu._lib.ssu_check_indices(ctypes.byref(args), None) == 0


def test_strided_pool_view(ref):
    """The pool may be one layer's view of a larger cache (slot stride larger
    than H*P*N); the state of other layers must stay untouched."""
    torch = gu.torch_mod()
    p = si.make_problem(H=4, P=64, N=128, batch=5, pool_slots=9, seed=1200)
    big = torch.randn(9, 3, 4, 64, 128, device="cuda")
    big[:, 1] = torch.from_numpy(p.pool).cuda()
    other = big[:, [0, 2]].clone()
    pool_view = big[:, 1]
    dp = gu.DeviceProblem(p, pool=pool_view)
    out = dp.run()
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), out, "strided pool")
    assert torch.equal(big[:, [0, 2]], other)


@pytest.mark.parametrize("H,P,N,G,bs", [
    (16, 64, 16, 1, 4096), (16, 64, 32, 1, 2048), (16, 64, 64, 1, 1024), (16, 64, 256, 1, 256),
    (16, 32, 128, 1, 1024), (16, 128, 128, 1, 256), (16, 64, 128, 2, 512), (16, 64, 128, 8, 512),
])
def test_other_shapes_at_bench_size(ref, H, P, N, G, bs):
    """The other-shape workloads at their measured size (256 MiB of state per
    call) in the launch configuration the library picks: every request
    against the oracle, untouched slots bitwise."""
    torch = gu.torch_mod()
    slots = bs + 16
    p = si.make_problem(H=H, P=P, N=N, G=G, batch=bs, pool_slots=slots, seed=900 + N + P + G, host_pool=False)
    pool = torch.empty((slots, H, P, N), device="cuda")
    si.draw_pool_on_device(pool, p.seed)
    dp = gu.DeviceProblem(p, pool=pool)
    backup = pool.clone()
    out = dp.run()
    torch.cuda.synchronize()
    sample = np.arange(bs)
    sl = torch.from_numpy(p.idx[sample].astype(np.int64)).cuda()
    sub_pool = backup[sl].cpu().numpy()
    r = ref.run(sub_pool, np.arange(len(sample), dtype=np.int32), p.x[sample], p.B[sample], p.C[sample],
                p.dt[sample], p.A, p.dt_bias, p.D)
    what = f"H{H} P{P} N{N} G{G} bs{bs}"
    gu.assert_state(pool[sl].cpu().numpy(), r["state"], what)
    gu.assert_out(gu.bits(out)[sample], r, what)
    mask = torch.ones(slots, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(p.idx.astype(np.int64)).cuda()] = False
    assert torch.equal(pool[mask].view(torch.int32), backup[mask].view(torch.int32)), what


def test_largest_sweep_point(ref):
    """H=128, batch 1024 (4 GiB of state per call) in the launch configuration
    the library picks: every request against the oracle, untouched slots
    bitwise, rerun bitwise."""
    torch = gu.torch_mod()
    H, bs = 128, 1024
    p = si.make_problem(H=H, P=64, N=128, batch=bs, pool_slots=bs + 64, seed=si.sweep_seed(H, bs),
                        host_pool=False)
    pool = torch.empty((bs + 64, H, 64, 128), device="cuda")
    si.draw_pool_on_device(pool, p.seed)
    dp = gu.DeviceProblem(p, pool=pool)
    backup = pool.clone()
    out = dp.run()
    torch.cuda.synchronize()
    sample = np.arange(bs)
    sl = torch.from_numpy(p.idx[sample].astype(np.int64)).cuda()
    before = backup[sl].cpu().numpy()
    after = pool[sl].cpu().numpy()
    sub_pool = before.copy()
    sub_idx = np.arange(len(sample), dtype=np.int32)
    r = ref.run(sub_pool, sub_idx, p.x[sample], p.B[sample], p.C[sample], p.dt[sample], p.A, p.dt_bias, p.D)
    gu.assert_state(after, r["state"], "H128 bs1024")
    gu.assert_out(gu.bits(out)[sample], r, "H128 bs1024")
    mask = torch.ones(bs + 64, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(p.idx.astype(np.int64)).cuda()] = False
    assert torch.equal(pool[mask].view(torch.int32), backup[mask].view(torch.int32))
    o1 = out.clone()
    s1 = pool[sl].clone()
    pool.copy_(backup)
    dp.run(out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(pool[sl].view(torch.int32), s1.view(torch.int32))


def test_nonfinite_values_stay_in_their_rows(ref):
    """NaN and infinity in the state, in x and in dt reach exactly the state
    elements and outputs the recurrence routes them to, with the oracle's IEEE
    class and sign, and every finite result keeps its tolerance: nothing
    spreads across rows, heads or requests (the row sums and the cross-lane
    reduction included)."""
    from . import tolerance as tol

    torch = gu.torch_mod()
    p = si.make_problem(H=2, P=64, N=128, batch=5, pool_slots=9, seed=1400)
    s = p.idx
    p.pool[s[0], 0, 5, 7] = np.nan       # one state element
    p.pool[s[1], 1, 10, 3] = np.inf      # infinities in two rows of one head
    p.pool[s[1], 1, 11, 4] = -np.inf
    P = p.headdim
    p.xbc[2, 0 * P + 20] = 0x7FC0        # NaN in x (request 2, head 0, row 20)
    p.xbc[3, 1 * P + 30] = 0x7F80        # +inf in x (request 3, head 1, row 30)
    p.dt[4, 0] = 0x7FC0                  # NaN step: the whole (request 4, head 0)
    before = p.pool.copy()
    dp = gu.DeviceProblem(p)
    out = dp.run()
    torch.cuda.synchronize()
    r = gu.oracle_step(ref, p, before.copy())

    got = dp.pool.cpu().numpy()[s].astype(np.float64)
    want = r["state"]
    for cls in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(cls(got), cls(want)), f"state class {cls.__name__}"
    assert np.isnan(want).any() and np.isinf(want).any()
    fin = np.isfinite(want)
    assert not tol.state_violations(got[fin], want[fin]).any(), "finite state"

    ob = gu.bits(out)
    g = tol.bf16_to_f64(ob)
    y = r["y"]
    for cls in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(cls(g), cls(y)), f"out class {cls.__name__}"
    assert np.isnan(y[4, 0]).all() and np.isfinite(y[4, 1]).all()
    fin = np.isfinite(y)
    fail, _ = tol.out_check(ob[fin], r["out"][fin], y[fin], r["tau"][fin])
    assert not fail.any(), "finite out"
    untouched = np.setdiff1d(np.arange(p.pool_slots), s)
    assert np.array_equal(dp.pool.cpu().numpy()[untouched].view(np.uint32), before[untouched].view(np.uint32))


@pytest.mark.parametrize("case", range(16))
def test_random_shapes(ref, case):
    """Seeded random shapes and options drawn together: d_state, headdim,
    heads, groups, batch, pool size, padding entries, int32 or int64 ids,
    softplus, dt_bias and D present or not, and the library's launch
    configuration or a random compiled one; every element against the oracle,
    untouched slots bitwise."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    rng = np.random.Generator(np.random.PCG64([88, case]))
    N = int(rng.choice([16, 32, 64, 128, 256]))
    P = 16 * int(rng.integers(1, 17))
    H = int(rng.integers(1, 25))
    G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
    per_unit = P * N * 4
    bs = int(rng.integers(1, max(2, min(40, (48 << 20) // (per_unit * H)) + 1)))
    slots = bs + int(rng.integers(0, 11))
    softplus = bool(rng.integers(0, 2))
    use_bias, use_D = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    p = si.make_problem(H=H, P=P, N=N, G=G, batch=bs, pool_slots=slots, seed=5000 + case, dt_softplus=softplus)
    if not softplus:
        # steps dt + dt_bias >= 0, as a step size is: a negative one makes the
        # decay exp(A * delta) grow and can overflow fp32
        p.dt = p.dt & np.uint16(0x7FFF)
        p.dt_bias = np.full(H, 0.01, dtype=np.float32)
    idx = p.idx.copy()
    if bs > 1 and rng.integers(0, 2):
        idx[int(rng.integers(0, bs))] = -1 if rng.integers(0, 2) else slots  # padding
    p.idx = idx
    tile = -1
    if rng.integers(0, 10) < 3:
        fits = [t["id"] for t in ssu.tiles() if t["dstate"] == N and ssu.tile_fits(t, H, P)]
        tile = int(rng.choice(fits))
    what = (f"case {case}: N {N} P {P} H {H} G {G} bs {bs} slots {slots} softplus {softplus} "
            f"bias {use_bias} D {use_D} tile {tile}")
    print(what, flush=True)
    dp = gu.DeviceProblem(p)
    ids = dp.idx.to(torch.int64) if rng.integers(0, 2) else dp.idx
    out = dp.run(tile=tile, use_bias=use_bias, use_D=use_D, idx=ids)
    torch.cuda.synchronize()
    gu.compare_full(ref, dp, p.pool.copy(), out, what, use_bias=use_bias, use_D=use_D)
