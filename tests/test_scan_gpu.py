"""The selective scan over a sequence (ssu_scan) against the CPU oracle.

Every output and every final state element is compared with the oracle's
fp64 scan under the scan rules of tests/tolerance.py, on the workloads of
ssu_inputs.SCAN_CONFIGS at full size (the oracle scans them in seconds), on
ragged lengths, other state counts and groups, every launch configuration,
unaligned (scalar-path) views and HIP graph replays. Chunkings whose chunks are
multiples of 512 tokens must agree bitwise with one launch over the whole
sequence (the state is carried in fp32 either way).
"""
import functools

import numpy as np
import pytest

import ssu_inputs as si

from . import gpu_util as gu
from . import tolerance as tol

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _io_tensor(bits, io, device="cuda"):
    torch = gu.torch_mod()
    dt = torch.float16 if io == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to(device)


class DeviceScan:
    """Device copies of a ScanProblem's operands (contiguous)."""

    def __init__(self, p: si.ScanProblem):
        torch = gu.torch_mod()
        self.p = p
        self.u = _io_tensor(p.u, p.io)
        self.delta = _io_tensor(p.delta, p.io)
        self.B = _io_tensor(p.B, p.io)
        self.C = _io_tensor(p.C, p.io)
        self.A = torch.from_numpy(p.A).cuda()
        self.D = torch.from_numpy(p.D).cuda()
        self.bias = torch.from_numpy(p.delta_bias).cuda()
        self.state0 = torch.from_numpy(p.state).cuda()

    def run(self, chunk=0, tile=-1, D=True, bias=True, views=None):
        import selective_state_update_amd as ssu

        torch = gu.torch_mod()
        v = dict(u=self.u, delta=self.delta, B=self.B, C=self.C)
        if views:
            v.update(views)
        state = self.state0.clone()
        out = ssu.selective_scan(v["u"], v["delta"], self.A, v["B"], v["C"], state,
                                 D=self.D if D else None, delta_bias=self.bias if bias else None,
                                 delta_softplus=self.p.delta_softplus, chunk=chunk, tile=tile)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy().view(np.uint16), state.cpu().numpy()


def oracle_scan(ref, p, D=True, bias=True):
    st = p.state.copy()
    return ref.scan(st, p.u, p.delta, p.A, p.B, p.C, p.D if D else None, p.delta_bias if bias else None,
                    delta_softplus=p.delta_softplus, io=p.io)


def check(p, out, state, r, what=""):
    rs, ro = tol.scan_error_ratios(out, state, r["y"], r["tau"], r["rho"], r["state"], r["err"], p.dstate, p.io)
    print(f"  {what}: worst state error {rs:.3f} eps*E (bound {tol.SCAN_STATE_C:g}), "
          f"worst out excess {ro:.4f} eps*(rho+N*tau) (bound {tol.SCAN_OUT_C:g})", flush=True)
    assert rs <= tol.SCAN_STATE_WATCH and ro <= tol.SCAN_OUT_WATCH, (
        f"{what}: error ratios {rs:.3f} / {ro:.4f} past the regression watch "
        f"{tol.SCAN_STATE_WATCH:g} / {tol.SCAN_OUT_WATCH:g}")
    bad_o = tol.scan_out_violations(out, r["y"], r["tau"], r["rho"], p.dstate, p.io)
    bad_s = tol.scan_state_violations(state, r["state"], r["err"])
    if bad_o.any():
        i = np.argwhere(bad_o)[0]
        raise AssertionError(f"{what}: {bad_o.sum()} outputs out of tolerance, first {tuple(i)}: "
                             f"gpu {tol.io_to_f64(out[tuple(i)], p.io)} ref {r['y'][tuple(i)]}")
    if bad_s.any():
        i = np.argwhere(bad_s)[0]
        raise AssertionError(f"{what}: {bad_s.sum()} states out of tolerance, first {tuple(i)}: "
                             f"gpu {state[tuple(i)]} ref {r['state'][tuple(i)]} err {r['err'][tuple(i)]}")


def _cfg(k):
    c = dict(si.SCAN_CONFIGS[k])
    name, chunk = c.pop("name"), c.pop("chunk")
    return name, chunk, c


@functools.lru_cache(maxsize=None)
def _config_case(k, zero_state):
    name, chunk, c = _cfg(k)
    p = si.make_scan_problem(**c, zero_state=zero_state)
    return name, chunk, p


@functools.lru_cache(maxsize=None)
def _config_ref(k, zero_state):
    import oracle

    _, _, p = _config_case(k, zero_state)
    return oracle_scan(oracle.get(), p)


@pytest.mark.parametrize("k", sorted(si.SCAN_CONFIGS))
@pytest.mark.parametrize("zero_state", [True, False], ids=["fresh", "carried"])
def test_scan_configs(k, zero_state):
    name, chunk, p = _config_case(k, zero_state)
    print(f"scan parity: {name} zero_state={zero_state}", flush=True)
    out, state = DeviceScan(p).run(chunk=chunk)
    check(p, out, state, _config_ref(k, zero_state), name)


def test_scan_chunk_invariance():
    """Chunks that are multiples of 512 tokens give bitwise the results of one
    launch, in the default configuration and in every configuration with 16
    tokens per lane (blocks of 512); other chunk sizes (including ragged ones)
    stay within tolerance."""
    import selective_state_update_amd as ssu

    name, _, p = _config_case(1, False)
    ds = DeviceScan(p)
    o0, s0 = ds.run(chunk=0)
    for chunk in (512, 1024, 1536, 4096):
        o, s = ds.run(chunk=chunk)
        assert np.array_equal(o, o0) and np.array_equal(s, s0), chunk
    for tile, tname in enumerate(ssu.scan_tiles()):
        if tname.startswith("scan_t16_"):
            for chunk in (512, 0):
                o, s = ds.run(chunk=chunk, tile=tile)
                assert np.array_equal(o, o0) and np.array_equal(s, s0), (tname, chunk)
    r = _config_ref(1, False)
    for chunk in (32, 64, 100, 256, 1000):
        o, s = ds.run(chunk=chunk)
        check(p, o, s, r, f"{name} chunk {chunk}")


def test_scan_every_tile():
    """Every launch configuration, on a small case with several blocks and a
    ragged tail, and with chunk sizes that do not fill a block."""
    import oracle
    import selective_state_update_amd as ssu

    p = si.make_scan_problem(2, 48, 16, 1337, 2, io="f16", seed=40, zero_state=False)
    r = oracle_scan(oracle.get(), p)
    ds = DeviceScan(p)
    for tile, name in enumerate(ssu.scan_tiles()):
        for chunk in (0, 200):
            o, s = ds.run(chunk=chunk, tile=tile)
            check(p, o, s, r, f"{name} chunk {chunk}")


@pytest.mark.parametrize("N", [1, 5, 17, 32, 48, 64])
def test_scan_every_tile_more_states(N):
    """Every launch configuration at d_state other than 16: below it (a
    partial round, the missing states staged as zeros) and above it (the
    staged and paired configurations then stage their rows in several rounds,
    the direct ones run several waves per channel), with a ragged tail and a
    chunk that splits blocks: within tolerance of the oracle, and the
    configurations with the same token segment bitwise equal to each other."""
    import oracle
    import selective_state_update_amd as ssu

    p = si.make_scan_problem(2, 32, N, 700, 2, io="bf16", seed=70 + N, zero_state=False)
    r = oracle_scan(oracle.get(), p)
    ds = DeviceScan(p)
    first = {}
    for tile, name in enumerate(ssu.scan_tiles()):
        seg = name.split("_")[1]
        for chunk in (0, 256):
            o, s = ds.run(chunk=chunk, tile=tile)
            check(p, o, s, r, f"N={N} {name} chunk {chunk}")
            key = (seg, chunk)
            if key not in first:
                first[key] = (name, o, s)
            else:
                n0, o0, s0 = first[key]
                assert np.array_equal(o, o0) and np.array_equal(s, s0), (name, n0, chunk)


@pytest.mark.parametrize("batch,dim,G,chunk,want", [
    (3, 1024, 1, 1024, "scan_t16_n16_pair_c8"),
    (3, 1028, 1, 1024, "scan_t16_n16_w1_c4"),
    (3, 1032, 2, 1024, "scan_t16_n16_w1_c4"),
    (3, 1026, 1, 1024, "scan_t16_n16"),
    (2, 1024, 1, 1024, "scan_t16_n16_w1_c4"),
    (3, 1024, 1, 512, "scan_t16_n16"),
])
def test_scan_default_rule_branches(batch, dim, G, chunk, want):
    """The default rule's branches: at chunk 1024 (two blocks) above 2048
    channels paired where a group's channels split into eights, staged where
    only into fours, direct otherwise, and staged at 2048 channels; at chunk
    512 (one block) direct. The default picks `want`, matches the oracle
    everywhere (a ragged last block, the chunk and one launch, which picks
    direct at 2048 channels), and equals the forced direct configuration
    bitwise."""
    import oracle
    import selective_state_update_amd as ssu

    p = si.make_scan_problem(batch, dim, 16, 1100, G, io="f16", seed=dim + G + batch, zero_state=False)
    ds = DeviceScan(p)
    a, _ = ssu.make_scan_args(ds.u, ds.delta, ds.A, ds.B, ds.C, ds.state0.clone(), ds.D, ds.bias)
    names = ssu.scan_tiles()
    assert names[ssu.scan_select_tile(a, chunk)] == want
    r = oracle_scan(oracle.get(), p)
    direct = names.index("scan_t16_n16")
    for c in (chunk, 0):
        o, s = ds.run(chunk=c)
        check(p, o, s, r, f"dim {dim} G {G} {want} chunk {c}")
        od, sd = ds.run(chunk=c, tile=direct)
        assert np.array_equal(o, od) and np.array_equal(s.view(np.uint32), sd.view(np.uint32)), c


@pytest.mark.parametrize("L", [1, 7, 63, 64, 65, 511, 513, 1000])
@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_scan_ragged_lengths(L, io):
    import oracle

    p = si.make_scan_problem(3, 40, 16, L, 1, io=io, seed=41 + L, zero_state=False)
    r = oracle_scan(oracle.get(), p)
    ds = DeviceScan(p)
    for chunk in (0, 64, 512):
        o, s = ds.run(chunk=chunk)
        check(p, o, s, r, f"L={L} {io} chunk {chunk}")


@pytest.mark.parametrize("N,G", [(1, 1), (4, 2), (16, 4), (17, 1), (32, 2), (48, 1), (64, 8)])
def test_scan_states_and_groups(N, G):
    """Other state counts (one wave up to 16 states, then one wave per 16) and
    B/C groups."""
    import oracle

    p = si.make_scan_problem(2, 64, N, 700, G, io="bf16", seed=50 + N + G, zero_state=False)
    r = oracle_scan(oracle.get(), p)
    o, s = DeviceScan(p).run(chunk=512)
    check(p, o, s, r, f"N={N} G={G}")


def test_scan_options():
    """Softplus off (positive steps), no D, no delta_bias."""
    import oracle

    p = si.make_scan_problem(2, 32, 16, 900, 1, io="f16", seed=60, zero_state=False, delta_softplus=False)
    # without the softplus the steps are delta + bias as given: keep them positive
    p.delta = si.io_bits(np.abs(si.io_values(p.delta, "f16")) * 0.05, "f16")
    p.delta_bias = np.full(p.dim, 0.01, dtype=np.float32)
    ref = oracle.get()
    for D, bias in ((True, True), (False, True), (True, False), (False, False)):
        r = oracle_scan(ref, p, D=D, bias=bias)
        o, s = DeviceScan(p).run(chunk=256, D=D, bias=bias)
        check(p, o, s, r, f"softplus off D={D} bias={bias}")


def test_scan_special_values():
    """A = 0 (no decay, the state is a running sum), A very negative (no
    memory), zero steps (softplus off, delta = bias = 0: state unchanged, out =
    C.h0 + D u) against the oracle."""
    import oracle

    ref = oracle.get()
    base = si.make_scan_problem(1, 32, 16, 600, 1, io="f16", seed=61, zero_state=False)
    cases = []
    p = si.make_scan_problem(1, 32, 16, 600, 1, io="f16", seed=61, zero_state=False)
    p.A = np.zeros_like(p.A)
    cases.append(("A=0", p, True))
    p = si.make_scan_problem(1, 32, 16, 600, 1, io="f16", seed=61, zero_state=False)
    p.A = np.full_like(p.A, -1e30)
    cases.append(("A=-1e30", p, True))
    p = si.make_scan_problem(1, 32, 16, 600, 1, io="f16", seed=61, zero_state=False, delta_softplus=False)
    p.delta = np.zeros_like(p.delta)
    cases.append(("zero steps", p, False))
    for what, p, bias in cases:
        r = oracle_scan(ref, p, bias=bias)
        o, s = DeviceScan(p).run(chunk=512, bias=bias)
        check(p, o, s, r, what)
        if what == "zero steps":
            assert np.array_equal(s, base.state)


def test_scan_unaligned_views():
    """Views that are not aligned for vector access (odd element offsets, row
    strides that are not multiples of 8) take the element-wise path, which
    must give bitwise the same results as the vector path."""
    torch = gu.torch_mod()
    p = si.make_scan_problem(2, 24, 16, 777, 2, io="bf16", seed=62, zero_state=False)
    ds = DeviceScan(p)
    o0, s0 = ds.run(chunk=512)

    def shifted(t):
        # same values, stored one element further into a wider buffer
        big = torch.zeros(t.shape[:-1] + (t.shape[-1] + 3,), dtype=t.dtype, device=t.device)
        big[..., 1:1 + t.shape[-1]] = t
        return big[..., 1:1 + t.shape[-1]]

    views = dict(u=shifted(ds.u), delta=shifted(ds.delta), B=shifted(ds.B), C=shifted(ds.C))
    o, s = ds.run(chunk=512, views=views)
    assert np.array_equal(o, o0) and np.array_equal(s, s0)
    o, s = ds.run(chunk=100, views=views)   # chunk starts not multiples of 8 either
    import oracle

    check(p, o, s, oracle_scan(oracle.get(), p), "unaligned chunk 100")


def test_scan_unaligned_views_every_tile():
    """Every launch configuration on views that are not aligned for vector
    access (the staged and paired kernels then stage B and C element by
    element): bitwise equal to the same configuration on aligned views, and
    configurations with the same token segment bitwise equal to each other."""
    torch = gu.torch_mod()
    import selective_state_update_amd as ssu

    p = si.make_scan_problem(2, 32, 20, 1300, 2, io="f16", seed=63, zero_state=False)
    ds = DeviceScan(p)

    def shifted(t):
        big = torch.zeros(t.shape[:-1] + (t.shape[-1] + 3,), dtype=t.dtype, device=t.device)
        big[..., 1:1 + t.shape[-1]] = t
        return big[..., 1:1 + t.shape[-1]]

    views = dict(u=shifted(ds.u), delta=shifted(ds.delta), B=shifted(ds.B), C=shifted(ds.C))
    first = {}
    for tile, name in enumerate(ssu.scan_tiles()):
        oa, sa = ds.run(chunk=512, tile=tile)
        ou, su = ds.run(chunk=512, tile=tile, views=views)
        assert np.array_equal(ou, oa) and np.array_equal(su.view(np.uint32), sa.view(np.uint32)), name
        seg = name.split("_")[1]
        if seg in first:
            n0, o0, s0 = first[seg]
            assert np.array_equal(oa, o0) and np.array_equal(sa.view(np.uint32), s0.view(np.uint32)), (name, n0)
        else:
            first[seg] = (name, oa, sa)
    import oracle

    check(p, first["t16"][1], first["t16"][2], oracle_scan(oracle.get(), p), "unaligned every tile")


def test_scan_batch_and_strided_state():
    """Several requests with a state that is a strided view into a larger
    buffer (rows of a state pool), and the output of one request unaffected by
    another's inputs."""
    import oracle
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    p = si.make_scan_problem(4, 32, 16, 530, 1, io="f16", seed=63, zero_state=False)
    r = oracle_scan(oracle.get(), p)
    ds = DeviceScan(p)
    pool = torch.full((9, 32, 16), 7.0, dtype=torch.float32, device="cuda")
    st = pool[1::2]  # rows 1, 3, 5, 7 of the pool: a non-contiguous view
    st.copy_(ds.state0)
    out = ssu.selective_scan(ds.u, ds.delta, ds.A, ds.B, ds.C, st, D=ds.D, delta_bias=ds.bias, chunk=512)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    check(p, o, st.cpu().numpy(), r, "strided state")
    assert np.all(pool[0::2].cpu().numpy() == 7.0)


def test_scan_empty():
    """batch 0 and length 0 are no-ops."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    p = si.make_scan_problem(2, 16, 16, 0, 1, io="f16", seed=64, zero_state=False)
    ds = DeviceScan(p)
    o, s = ds.run(chunk=512)
    assert o.size == 0 and np.array_equal(s, p.state)
    act = torch.zeros((0, 16, 5), dtype=torch.float16, device="cuda")
    bc = torch.zeros((0, 1, 16, 5), dtype=torch.float16, device="cuda")
    state = torch.zeros((0, 16, 16), dtype=torch.float32, device="cuda")
    out = ssu.selective_scan(act, act, ds.A, bc, bc, state, chunk=512)
    assert out.shape == (0, 16, 5)


@pytest.mark.parametrize("tile_name", ["default", "scan_t16_n16_w1_c4", "scan_t16_n16_pair_c8"])
def test_scan_graph_replays(tile_name):
    """The chunked scan captured in a HIP graph, in the default configuration
    and forced to the staged and paired kernels: every replay (state reset
    between replays by an eager copy) matches the eager default result
    bitwise."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    name, chunk, p = _config_case(0, False)
    tile = -1 if tile_name == "default" else ssu.scan_tiles().index(tile_name)
    ds = DeviceScan(p)
    o_ref, s_ref = ds.run(chunk=chunk)
    state = ds.state0.clone()
    args, out = ssu.make_scan_args(ds.u, ds.delta, ds.A, ds.B, ds.C, state, ds.D, ds.bias)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ssu.scan_launch(args, chunk, tile, stream=s)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ssu.scan_launch(args, chunk, tile, stream=s)
    for rep in range(3):
        state.copy_(ds.state0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(o, o_ref) and np.array_equal(state.cpu().numpy(), s_ref), rep


def test_scan_long_sequence():
    """A sequence of about a million tokens (ragged, several launches of
    2^18 tokens and one launch): 64-bit token offsets and many blocks, every
    output and the final state against the oracle."""
    import oracle

    L = 1_000_003
    p = si.make_scan_problem(1, 4, 16, L, 1, io="bf16", seed=65, zero_state=False)
    r = oracle_scan(oracle.get(), p)
    ds = DeviceScan(p)
    for chunk in (1 << 18, 0):
        o, s = ds.run(chunk=chunk)
        check(p, o, s, r, f"L={L} chunk {chunk}")


@pytest.mark.parametrize("case", range(12))
def test_scan_random_shapes(case):
    """Seeded random shapes: batch, dim, states, groups, length, activation
    type, chunk, softplus and which optional parameters are present drawn
    together, each against the oracle."""
    import oracle

    rng = np.random.Generator(np.random.PCG64([77, case]))
    N = int(rng.integers(1, 65))
    G = int(rng.choice([1, 2, 4]))
    dim = G * int(rng.integers(1, 24))
    batch = int(rng.integers(1, 4))
    L = int(rng.integers(1, 3000))
    io = str(rng.choice(["f16", "bf16"]))
    softplus = bool(rng.integers(0, 2))
    chunk = int(rng.choice([0, 64, 100, 512, 777]))
    p = si.make_scan_problem(batch, dim, N, L, G, io=io, seed=1000 + case, zero_state=bool(rng.integers(0, 2)),
                             delta_softplus=softplus)
    if not softplus:
        p.delta = si.io_bits(np.abs(si.io_values(p.delta, io)) * 0.05, io)
        p.delta_bias = np.full(dim, 0.01, dtype=np.float32)
    D, bias = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    r = oracle_scan(oracle.get(), p, D=D, bias=bias)
    o, s = DeviceScan(p).run(chunk=chunk, D=D, bias=bias)
    check(p, o, s, r, f"case {case}: batch {batch} dim {dim} N {N} G {G} L {L} {io} chunk {chunk} "
                      f"softplus {softplus} D {D} bias {bias}")


def _same_nonfinite(gpu, ref, what):
    """Finite exactly where the oracle is; NaN where it is NaN; where it is
    infinite, the same infinity or NaN. (A state that has become infinite
    stays infinite in the sequential oracle, since every decay is positive; the
    kernel composes a block's decays into one product, which underflows to 0
    for fast-decaying states, and 0 * inf is NaN.)"""
    g = np.asarray(gpu, dtype=np.float64)
    assert np.array_equal(np.isfinite(g), np.isfinite(ref)), f"{what}: finite pattern"
    assert np.isnan(g[np.isnan(ref)]).all(), f"{what}: NaN"
    for sign in (np.isposinf, np.isneginf):
        m = sign(ref)
        assert (sign(g[m]) | np.isnan(g[m])).all(), f"{what}: {sign.__name__}"


def test_scan_nonfinite_inputs():
    """Infinite and NaN activations reach exactly the outputs and states the
    recurrence routes them to: a step of -inf (softplus 0) is the identity, a
    step of +inf wipes the channel's memory and makes it non-finite from that
    token on, a NaN input poisons its channel from that token on; earlier
    tokens and other channels keep their tolerance."""
    import oracle

    ref = oracle.get()
    p = si.make_scan_problem(1, 8, 16, 1100, 1, io="f16", seed=63, zero_state=False)
    p.delta[0, 1, 100] = 0x7C00   # +inf
    p.delta[0, 2, 300] = 0xFC00   # -inf
    p.u[0, 3, 500] = 0x7E00       # NaN
    r = oracle_scan(ref, p)
    o, s = DeviceScan(p).run(chunk=512)
    g = tol.io_to_f64(o, p.io)
    y, st = r["y"], r["state"]
    _same_nonfinite(g, y, "out")
    _same_nonfinite(s, st, "state")
    # where they land
    assert np.isfinite(y[0, 1, :100]).all() and not np.isfinite(y[0, 1, 100:]).any()
    assert np.isinf(st[0, 1]).all()
    assert np.isfinite(y[0, 2]).all() and np.isfinite(st[0, 2]).all()
    assert np.isfinite(y[0, 3, :500]).all() and np.isnan(y[0, 3, 500:]).all() and np.isnan(st[0, 3]).all()
    others = [0, 4, 5, 6, 7]
    assert np.isfinite(y[0, others]).all() and np.isfinite(st[0, others]).all()
    fin = np.isfinite(y)
    bad = tol.scan_out_violations(o[fin], y[fin], r["tau"][fin], r["rho"][fin], p.dstate, p.io)
    assert not bad.any(), "finite outputs"
    fin = np.isfinite(st)
    bad = tol.scan_state_violations(s[fin], st[fin], r["err"][fin])
    assert not bad.any(), "finite states"


def test_scan_many_requests():
    """The saturation workload: 16 requests x 1024 channels, d_state 16, 4096
    fp16 tokens, static chunk 512. Chunk 512 is bitwise equal to one launch,
    and every output and final state matches the oracle's scan."""
    import oracle

    p = si.make_scan_problem(16, 1024, 16, 4096, io="f16", seed=17, zero_state=False)
    ds = DeviceScan(p)
    out512, st512 = ds.run(chunk=512)
    out1, st1 = ds.run(chunk=0)
    assert np.array_equal(out512, out1), "chunk 512 and one launch differ (out)"
    assert np.array_equal(st512.view(np.uint32), st1.view(np.uint32)), "chunk 512 and one launch differ (state)"
    r = oracle_scan(oracle.get(), p)
    check(p, out512, st512, r, "16 requests x 1024 channels")
