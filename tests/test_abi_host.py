"""libssu's C ABI on the host: it loads, exports what include/ssu.h declares,
and rejects bad arguments before touching the GPU.

No test here launches a kernel: every ssu_update call below carries at least
one invalid field (or batch 0), so the library returns before any HIP call.
The pointer values are never dereferenced on the host.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssu.h")


@pytest.fixture(scope="module")
def ssu():
    import selective_state_update_amd as m

    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssu_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ssu_create", "ssu_update", "ssu_destroy", "ssu_status_string", "ssu_check_indices"):
        assert n in names


def test_library_exports_every_declared_symbol(ssu):
    lib = ctypes.CDLL(ssu.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", ssu.library_path()], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT (ssu_[a-z_0-9]+)$", out.stdout, flags=re.M))
        assert set(declared_functions()) <= exported


def test_abi_version(ssu):
    text = open(HEADER).read()
    want = int(re.search(r"#define SSU_ABI_VERSION (\d+)", text).group(1))
    assert ssu.abi_version() == want


def test_status_strings(ssu):
    for code, name in ssu.STATUS_NAMES.items():
        assert ssu._lib.ssu_status_string(code).decode() == name
    assert ssu._lib.ssu_status_string(99).decode() == "SSU_ERR_UNKNOWN"


def test_struct_layout_matches_header(ssu):
    # ssu_view: pointer, two int32, four int64
    assert ctypes.sizeof(ssu.View) == 8 + 4 + 4 + 32
    assert ctypes.sizeof(ssu.Config) == 8 * 4
    assert ctypes.sizeof(ssu.Args) == 16 + 10 * ctypes.sizeof(ssu.View)
    assert ctypes.sizeof(ssu.TileDesc) == 7 * 4 + 48


def _create(ssu, **kw):
    cfg = dict(nheads=16, headdim=64, dstate=128, ngroups=1, dt_softplus=1, tile=-1, device=-1, reserved=0)
    cfg.update(kw)
    c = ssu.Config(**cfg)
    h = ctypes.c_void_p()
    st = ssu._lib.ssu_create(ctypes.byref(c), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,code", [
    (dict(nheads=0), 1),
    (dict(ngroups=3), 1),
    (dict(ngroups=0), 1),
    (dict(headdim=0), 1),
    (dict(dstate=100), 2),
    (dict(dstate=512), 2),
    (dict(headdim=24), 2),
    (dict(headdim=512), 2),
    (dict(dt_softplus=2), 1),
    (dict(tile=100000), 1),
    (dict(tile=-2), 1),
    (dict(device=-5), 1),
    (dict(reserved=1), 1),
])
def test_create_rejects(ssu, kw, code):
    st, h = _create(ssu, **kw)
    assert st == code, ssu._lib.ssu_last_error()
    assert not h.value
    assert ssu._lib.ssu_last_error().decode()


def test_create_rejects_tile_for_other_dstate(ssu):
    t = ssu.tiles()
    wrong = next(x["id"] for x in t if x["dstate"] != 128)
    st, h = _create(ssu, tile=wrong)
    assert st == 1 and not h.value


def test_create_env_override(ssu, monkeypatch):
    monkeypatch.setenv("SSU_TILE", "not-a-number")
    st, _ = _create(ssu)
    assert st == 1
    t = next(x["id"] for x in ssu.tiles() if x["dstate"] == 128)
    monkeypatch.setenv("SSU_TILE", str(t))
    st, h = _create(ssu)
    assert st == 0
    assert ssu._lib.ssu_select_tile(h, 512) == t
    ssu._lib.ssu_destroy(h)


def test_destroy_null_is_noop(ssu):
    ssu._lib.ssu_destroy(None)


def test_tiles_are_described(ssu):
    t = ssu.tiles()
    assert len(t) == ssu._lib.ssu_tile_count() > 0
    names = [x["name"] for x in t]
    assert len(set(names)) == len(names)
    for x in t:
        assert x["rows_per_group"] == x["rows_per_wave"] * x["waves"]
        assert x["groups_per_cu"] == 0 or (x["nontemporal"] and x["xcd_remap"])
        assert x["dstate"] in (16, 32, 64, 128, 256)
    d = ssu.TileDesc()
    assert ssu._lib.ssu_tile_info(len(t), ctypes.byref(d)) == 1
    assert ssu._lib.ssu_tile_info(0, None) == 1


@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("P", [16, 64, 80, 256])
def test_select_tile_fits_shape(ssu, N, P):
    st, h = _create(ssu, dstate=N, headdim=P)
    assert st == 0
    t = ssu.tiles()
    for bs in (1, 8, 128, 512, 1024):
        i = ssu._lib.ssu_select_tile(h, bs)
        assert i >= 0
        assert t[i]["dstate"] == N and ssu.tile_fits(t[i], 16, P)
    ssu._lib.ssu_destroy(h)


@pytest.mark.parametrize("H", [1, 4, 12, 16])
@pytest.mark.parametrize("N,P", [(16, 64), (32, 64), (16, 128), (128, 64)])
def test_forced_tile_accepted_iff_it_fits(ssu, H, N, P):
    """ssu_create takes a forced launch configuration exactly when tile_fits
    says it serves H heads of headdim P (rows per group dividing P, or waves
    of one whole head each that split the heads evenly)."""
    t = ssu.tiles()
    multi = 0
    for x in t:
        if x["dstate"] != N:
            continue
        st, h = _create(ssu, nheads=H, headdim=P, dstate=N, tile=x["id"])
        fits = ssu.tile_fits(x, H, P)
        assert (st == 0) == fits, (x["name"], H, P, st)
        multi += fits and x["rows_per_group"] > P
        if st == 0:
            ssu._lib.ssu_destroy(h)
    if (N, P, H) in ((16, 64, 16), (32, 64, 16)):
        assert multi > 0  # groups of several whole heads exist for these shapes


@pytest.mark.parametrize("bs,K,name", [
    (512, 1, "n128_r8_w1_nt_xcd_g12"), (128, 1, "n128_r8_w1_nt_xcd_g12"), (64, 1, "n128_r8_w1_nt_xcd_g12"),
    (32, 1, "n128_r32_w2_nt_xcd"), (16, 1, "n128_r16_w2_nt_xcd"), (8, 1, "n128_r8_w1_nt_xcd"),
    (4, 1, "n128_r4_w1_nt_xcd"), (1, 1, "n128_r4_w1_nt_xcd"),
    (512, 2, "n128_r8_w1_nt_xcd_g14"), (512, 3, "n128_r8_w1_nt_xcd_g20"), (512, 4, "n128_r8_w1_nt_xcd"),
    (256, 2, "n128_r8_w1_nt_xcd_g14"), (128, 2, "n128_r8_w1_nt_xcd"), (128, 3, "n128_r8_w1_nt_xcd"),
    (512, 8, "n128_r16_w1_nt_xcd"), (512, 16, "n128_r16_w2_nt_xcd"),
    (128, 4, "n128_r16_w1_nt_xcd"), (128, 16, "n128_r16_w2_nt_xcd"),
])
def test_launch_rule_at_the_swept_points(ssu, bs, K, name):
    """The launch table picks, at H16 P64 N128, the configurations the tile
    sweeps measured fastest (or within 1% of it)."""
    st, h = _create(ssu)
    assert st == 0
    i = ssu._lib.ssu_select_tile_tokens(h, bs, K) if K > 1 else ssu._lib.ssu_select_tile(h, bs)
    assert ssu.tiles()[i]["name"] == name
    ssu._lib.ssu_destroy(h)


@pytest.mark.parametrize("N", [16, 32, 64, 256])
@pytest.mark.parametrize("P", [16, 64, 256])
def test_select_tile_tokens_fits_shape(ssu, N, P):
    st, h = _create(ssu, dstate=N, headdim=P)
    assert st == 0
    t = ssu.tiles()
    for bs in (1, 8, 128, 512, 1024, 4096):
        for K in (2, 3, 4, 8, 16, 64):
            i = ssu._lib.ssu_select_tile_tokens(h, bs, K)
            assert i >= 0
            assert t[i]["dstate"] == N and ssu.tile_fits(t[i], 16, P)
    ssu._lib.ssu_destroy(h)


# ---------------------------------------------------------------- ssu_update --
FAKE = 0x7F0000000000  # 256-byte aligned fake device address, never dereferenced


def _good_args(ssu, bs=4, H=16, P=64, N=128, G=1):
    a = ssu.Args()
    a.batch, a.reserved, a.pool_slots = bs, 0, 8

    def v(off, dtype, strides):
        x = ssu.View()
        x.ptr = FAKE + off
        x.dtype = dtype
        x.reserved = 0
        for i, s in enumerate(strides):
            x.stride[i] = s
        return x

    row = H * P + 2 * G * N
    a.state = v(0, ssu.SSU_F32, (H * P * N, P * N, N, 1))
    a.idx = v(0x1000, ssu.SSU_I32, (1,))
    a.x = v(0x2000, ssu.SSU_BF16, (row, P, 1))
    a.B = v(0x2000 + 2 * H * P, ssu.SSU_BF16, (row, N, 1))
    a.C = v(0x2000 + 2 * (H * P + G * N), ssu.SSU_BF16, (row, N, 1))
    a.dt = v(0x3000, ssu.SSU_BF16, (H, 1, 0))
    a.dt_bias = v(0x4000, ssu.SSU_F32, (1, 0))
    a.A = v(0x5000, ssu.SSU_F32, (1, 0, 0))
    a.D = v(0x6000, ssu.SSU_F32, (1, 0))
    a.out = v(0x7000, ssu.SSU_BF16, (H * P, P, 1))
    return a


def _break(a, field, what, value):
    v = getattr(a, field)
    if what == "ptr":
        v.ptr = value
    elif what == "dtype":
        v.dtype = value
    elif what == "reserved":
        v.reserved = value
    else:
        v.stride[int(what)] = value
    setattr(a, field, v)


BAD = [
    ("state", "ptr", None, 1), ("idx", "ptr", None, 1), ("x", "ptr", None, 1), ("B", "ptr", None, 1),
    ("C", "ptr", None, 1), ("dt", "ptr", None, 1), ("A", "ptr", None, 1), ("out", "ptr", None, 1),
    ("state", "dtype", 1, 1), ("idx", "dtype", 0, 1), ("x", "dtype", 0, 1), ("B", "dtype", 2, 1),
    ("dt", "dtype", 0, 1), ("A", "dtype", 1, 1), ("D", "dtype", 1, 1), ("dt_bias", "dtype", 1, 1),
    ("out", "dtype", 0, 1), ("x", "reserved", 7, 1),
    ("state", "3", 2, 2), ("idx", "0", 2, 2), ("x", "2", 2, 2), ("out", "2", 2, 2), ("B", "2", 2, 2),
    ("C", "2", 3, 2), ("dt", "2", 1, 2), ("dt_bias", "1", 1, 2), ("A", "1", 1, 2), ("A", "2", 1, 2),
    ("D", "1", 1, 2), ("x", "0", -1280, 1),
    ("state", "ptr", FAKE + 8, 3), ("state", "0", 131070, 3), ("state", "2", 130, 3),
    ("B", "ptr", FAKE + 0x2000 + 2050, 3), ("C", "0", 1282, 3), ("x", "ptr", FAKE + 0x2002, 3),
    ("x", "1", 63, 3), ("dt", "ptr", FAKE + 0x3001, 3),
]


@pytest.mark.parametrize("field,what,value,code", BAD, ids=[f"{b[0]}.{b[1]}={b[2]}" for b in BAD])
def test_update_rejects_before_launch(ssu, field, what, value, code):
    st, h = _create(ssu)
    assert st == 0
    a = _good_args(ssu)
    _break(a, field, what, value)
    got = ssu._lib.ssu_update(h, ctypes.byref(a), None)
    assert got == code, (got, ssu._lib.ssu_last_error())
    ssu._lib.ssu_destroy(h)


def test_update_size_errors(ssu):
    st, h = _create(ssu)
    a = _good_args(ssu)
    a.batch = -1
    assert ssu._lib.ssu_update(h, ctypes.byref(a), None) == 1
    a = _good_args(ssu)
    a.pool_slots = -1
    assert ssu._lib.ssu_update(h, ctypes.byref(a), None) == 1
    a = _good_args(ssu)
    a.reserved = 3
    assert ssu._lib.ssu_update(h, ctypes.byref(a), None) == 1
    assert ssu._lib.ssu_update(None, ctypes.byref(a), None) == 1
    assert ssu._lib.ssu_update(h, None, None) == 1
    ssu._lib.ssu_destroy(h)


def test_batch_zero_is_a_noop(ssu):
    st, h = _create(ssu)
    a = ssu.Args()  # all pointers NULL: nothing may be read
    a.batch = 0
    assert ssu._lib.ssu_update(h, ctypes.byref(a), None) == 0
    assert ssu._lib.ssu_check_indices(ctypes.byref(a), None) == 0
    ssu._lib.ssu_destroy(h)


def test_check_indices_rejects_bad_views(ssu):
    a = _good_args(ssu)
    a.idx.ptr = None
    assert ssu._lib.ssu_check_indices(ctypes.byref(a), None) == 1
    a = _good_args(ssu)
    a.idx.dtype = ssu.SSU_F32
    assert ssu._lib.ssu_check_indices(ctypes.byref(a), None) == 1
    a = _good_args(ssu)
    a.batch = -2
    assert ssu._lib.ssu_check_indices(ctypes.byref(a), None) == 1


def test_python_binding_validates_shapes(ssu):
    import torch

    h = ssu.Handle(2, 64, 128)
    st = torch.zeros(4, 2, 64, 128)
    x = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    B = torch.zeros(3, 1, 128, dtype=torch.bfloat16)
    idx = torch.zeros(3, dtype=torch.int32)
    dt = torch.zeros(3, 2, dtype=torch.bfloat16)
    A = torch.zeros(2)
    out = torch.empty(3, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        h.make_args(st, idx, x[:, :1], B, B, dt, A, out=out)
    with pytest.raises(ValueError):
        h.make_args(st, idx, x, B[:, :, :64], B, dt, A, out=out)
    with pytest.raises(ValueError, match="GPU"):
        h.make_args(st, idx, x, B, B, dt, A, out=out)
    with pytest.raises(ssu.SSUError):
        ssu.Handle(2, 64, 100)


# ---------------------------------------------------------- ssu_update_tokens --
def _good_tokens_args(ssu, bs=4, T=3, H=16, P=64, N=128, G=1):
    a = ssu.TokensArgs()
    a.batch, a.ntokens, a.pool_slots = bs, T, 8

    def v(off, dtype, strides):
        x = ssu.View()
        x.ptr = FAKE + off
        x.dtype = dtype
        x.reserved = 0
        for i, s in enumerate(strides):
            x.stride[i] = s
        return x

    row = H * P + 2 * G * N
    a.state = v(0, ssu.SSU_F32, (H * P * N, P * N, N, 1))
    a.idx = v(0x1000, ssu.SSU_I32, (1,))
    a.x = v(0x2000, ssu.SSU_BF16, (T * row, row, P, 1))
    a.B = v(0x2000 + 2 * H * P, ssu.SSU_BF16, (T * row, row, N, 1))
    a.C = v(0x2000 + 2 * (H * P + G * N), ssu.SSU_BF16, (T * row, row, N, 1))
    a.dt = v(0x3000, ssu.SSU_BF16, (T * H, H, 1, 0))
    a.dt_bias = v(0x4000, ssu.SSU_F32, (1, 0))
    a.A = v(0x5000, ssu.SSU_F32, (1, 0, 0))
    a.D = v(0x6000, ssu.SSU_F32, (1, 0))
    a.out = v(0x7000, ssu.SSU_BF16, (T * H * P, H * P, P, 1))
    return a


TOKENS_BAD = [
    ("ntokens", 0, 1), ("ntokens", -3, 1), ("ntokens", 1025, 1),
    ("x.stride1", 1281, 3), ("B.stride1", 1282, 3), ("dt.stride3", 1, 2), ("x.stride3", 2, 2),
    ("out.stride3", 0, 2), ("C.stride3", 2, 2), ("x.ptr", None, 1), ("out.dtype", 0, 1),
]


@pytest.mark.parametrize("what,value,code", TOKENS_BAD, ids=[f"{b[0]}={b[1]}" for b in TOKENS_BAD])
def test_update_tokens_rejects_before_launch(ssu, what, value, code):
    st, h = _create(ssu)
    a = _good_tokens_args(ssu)
    if what == "ntokens":
        a.ntokens = value
    else:
        field, attr = what.split(".")
        v = getattr(a, field)
        if attr == "ptr":
            v.ptr = value
        elif attr == "dtype":
            v.dtype = value
        else:
            v.stride[int(attr[-1])] = value
        setattr(a, field, v)
    got = ssu._lib.ssu_update_tokens(h, ctypes.byref(a), None)
    assert got == code, (got, ssu._lib.ssu_last_error())
    ssu._lib.ssu_destroy(h)


def test_update_tokens_batch_zero_and_nulls(ssu):
    st, h = _create(ssu)
    a = ssu.TokensArgs()
    a.batch, a.ntokens = 0, 4
    assert ssu._lib.ssu_update_tokens(h, ctypes.byref(a), None) == 0
    assert ssu._lib.ssu_update_tokens(None, ctypes.byref(a), None) == 1
    assert ssu._lib.ssu_update_tokens(h, None, None) == 1
    a.batch = -1
    assert ssu._lib.ssu_update_tokens(h, ctypes.byref(a), None) == 1
    ssu._lib.ssu_destroy(h)


def test_tokens_struct_layout(ssu):
    assert ctypes.sizeof(ssu.TokensArgs) == 16 + 10 * ctypes.sizeof(ssu.View)
    text = open(HEADER).read()
    assert int(re.search(r"#define SSU_MAX_TOKENS (\d+)", text).group(1)) == 1024


# ------------------------------------------------------------ ssu_copy_blocks --
def test_copy_blocks_validation(ssu):
    B = ssu.BlockTensor
    lib = ssu._lib
    good = B(FAKE, 4096, 4096, 8)
    ids = ctypes.c_void_p(FAKE + 0x100000)

    def call(t, n=1, nreqs=2, tile=-1, src=ids, dst=ids):
        arr = (B * max(1, n))(*([t] * max(1, n)))
        return lib.ssu_copy_blocks(arr, n, src, dst, nreqs, tile, None)

    assert call(good, nreqs=0) == 0          # no work: nothing read
    assert call(good, n=0) == 0
    assert call(good, nreqs=-1) == 1
    assert call(good, n=-1) == 1
    assert call(good, tile=10 ** 6) == 1
    assert call(good, src=None) == 1
    assert call(B(None, 4096, 4096, 8)) == 1
    assert call(B(FAKE + 8, 4096, 4096, 8)) == 3
    assert call(B(FAKE, 4100, 4096, 8)) == 3
    assert call(B(FAKE, 4096, 4088, 8)) == 3
    assert call(B(FAKE, 4096, 8192, 8)) == 1  # blocks overlap
    assert call(B(FAKE, 4096, -16, 8)) == 1
    assert lib.ssu_copy_tile_count() > 0
    assert lib.ssu_copy_tile_name(0).decode().startswith("copy_")
    assert lib.ssu_copy_tile_name(-1) == b""
    names = [lib.ssu_copy_tile_name(i).decode() for i in range(lib.ssu_copy_tile_count())]
    assert len(set(names)) == len(names) and "copy_u2_xcd" in names


def test_copy_blocks_checks_every_group_before_launching(ssu):
    """More than 32 tensors take one launch per 32; a size error in a later
    group is reported before the first launch (here, with no GPU, a launch
    attempt would return SSU_ERR_HIP instead)."""
    B = ssu.BlockTensor
    ids = ctypes.c_void_p(FAKE + 0x100000)
    small = B(FAKE, 4096, 4096, 8)
    huge = B(FAKE, 1 << 40, 1 << 40, 1)   # 2^27 chunks of 8 KiB per request
    ts = [small] * 32 + [huge] + [small] * 7
    arr = (B * len(ts))(*ts)
    assert ssu._lib.ssu_copy_blocks(arr, len(ts), ids, ids, 32, -1, None) == 2  # 2^32 workgroups
    assert "2^31" in ssu._lib.ssu_last_error().decode()


# ------------------------------------------------------------------- ssu_scan --
def _scan_args(ssu, batch=1, dim=32, N=16, G=1, L=100, io=None, softplus=1):
    """ScanArgs over fake device addresses, contiguous layouts; tests change one
    field to something invalid so the call returns before any HIP call."""
    io = ssu.SSU_F16 if io is None else io
    a = ssu.ScanArgs()
    a.batch, a.dim, a.dstate, a.ngroups, a.seqlen = batch, dim, N, G, L
    a.delta_softplus, a.reserved = softplus, 0

    def view(off, tag, strides):
        v = ssu.View()
        v.ptr = FAKE + off
        v.dtype = tag
        for i, s_ in enumerate(strides):
            v.stride[i] = s_
        return v

    a.state = view(0x0, ssu.SSU_F32, (dim * N, N, 1))
    a.u = view(0x100000, io, (dim * L, L, 1))
    a.delta = view(0x200000, io, (dim * L, L, 1))
    a.B = view(0x300000, io, (G * N * L, N * L, L, 1))
    a.C = view(0x400000, io, (G * N * L, N * L, L, 1))
    a.A = view(0x500000, ssu.SSU_F32, (N, 1))
    a.D = view(0x600000, ssu.SSU_F32, (1,))
    a.delta_bias = view(0x700000, ssu.SSU_F32, (1,))
    a.out = view(0x800000, io, (dim * L, L, 1))
    return a


def test_scan_struct_layout(ssu):
    assert ctypes.sizeof(ssu.ScanArgs) == 32 + 9 * ctypes.sizeof(ssu.View)
    assert ssu.ScanArgs.state.offset == 32


def _scan_call(ssu, a, chunk=512, tile=-1):
    return ssu._lib.ssu_scan(ctypes.byref(a), chunk, tile, None)


@pytest.mark.parametrize("what,mutate,code", [
    ("negative dim", lambda a, s: setattr(a, "dim", -1), 1),
    ("zero dstate", lambda a, s: setattr(a, "dstate", 0), 1),
    ("dstate > 64", lambda a, s: setattr(a, "dstate", 65), 2),
    ("ngroups does not divide dim", lambda a, s: setattr(a, "ngroups", 3), 1),
    ("negative seqlen", lambda a, s: setattr(a, "seqlen", -5), 1),
    ("softplus flag", lambda a, s: setattr(a, "delta_softplus", 2), 1),
    ("null state", lambda a, s: setattr(a.state, "ptr", None), 1),
    ("null A", lambda a, s: setattr(a.A, "ptr", None), 1),
    ("null u", lambda a, s: setattr(a.u, "ptr", None), 1),
    ("null out", lambda a, s: setattr(a.out, "ptr", None), 1),
    ("state not f32", lambda a, s: setattr(a.state, "dtype", s.SSU_BF16), 1),
    ("A not f32", lambda a, s: setattr(a.A, "dtype", s.SSU_F16), 1),
    ("D not f32", lambda a, s: setattr(a.D, "dtype", s.SSU_BF16), 1),
    ("u not 16-bit", lambda a, s: setattr(a.u, "dtype", s.SSU_F32), 1),
    ("B dtype differs from u", lambda a, s: setattr(a.B, "dtype", s.SSU_BF16), 1),
    ("state's dstate axis strided", lambda a, s: a.state.stride.__setitem__(2, 2), 2),
    ("u's token axis strided", lambda a, s: a.u.stride.__setitem__(2, 2), 2),
    ("C's token axis strided", lambda a, s: a.C.stride.__setitem__(3, 0), 2),
    ("out's token axis strided", lambda a, s: a.out.stride.__setitem__(2, 3), 2),
    ("state misaligned", lambda a, s: setattr(a.state, "ptr", FAKE + 2), 3),
    ("u misaligned", lambda a, s: setattr(a.u, "ptr", FAKE + 0x100001), 3),
    ("batch * dim >= 2^31", lambda a, s: (setattr(a, "batch", 1 << 20), setattr(a, "dim", 1 << 12)), 2),
    ("reserved field", lambda a, s: setattr(a, "reserved", 1), 1),
    ("view reserved field", lambda a, s: setattr(a.B, "reserved", 7), 1),
    ("negative state stride", lambda a, s: a.state.stride.__setitem__(1, -16), 1),
    ("negative u stride", lambda a, s: a.u.stride.__setitem__(0, -100), 1),
    ("negative B stride", lambda a, s: a.B.stride.__setitem__(2, -100), 1),
    ("negative A stride", lambda a, s: a.A.stride.__setitem__(0, -16), 1),
    ("D strided", lambda a, s: a.D.stride.__setitem__(0, 2), 2),
    ("delta_bias strided", lambda a, s: a.delta_bias.stride.__setitem__(0, 0), 2),
])
def test_scan_rejects_before_launch(ssu, what, mutate, code):
    a = _scan_args(ssu)
    mutate(a, ssu)
    assert _scan_call(ssu, a) == code, what
    assert ssu._lib.ssu_last_error().decode().startswith("ssu_scan"), what


def test_scan_other_rejections(ssu):
    a = _scan_args(ssu)
    assert _scan_call(ssu, a, chunk=-1) == 1
    assert _scan_call(ssu, a, tile=ssu._lib.ssu_scan_tile_count()) == 1
    assert _scan_call(ssu, a, tile=-2) == 1
    assert ssu._lib.ssu_scan_tile_count() == len(ssu.scan_tiles()) == 28
    assert ssu._lib.ssu_scan_tile_name(0).decode().startswith("scan_")
    assert ssu._lib.ssu_scan_tile_name(99) == b""


@pytest.mark.parametrize("prefix", ["scan_t16_n16_w1_c4", "scan_t16_n16_pair_c8"])
def test_scan_staged_needs_32bit_row_offsets(ssu, prefix):
    """A launch configuration that stages B and C rows in LDS (staged and
    paired) addresses its staging pieces as 32-bit byte offsets from a row
    pointer: B or C state strides of 2^30 / 64 elements or more are refused for
    it before any launch (the default then picks the direct kernel, which takes
    64-bit addresses)."""
    names = ssu.scan_tiles()
    staged = next(i for i, n in enumerate(names) if n.startswith(prefix))
    a = _scan_args(ssu, dim=32)
    a.B.stride[2] = (1 << 30) // 64
    assert _scan_call(ssu, a, tile=staged) == 2
    err = ssu._lib.ssu_last_error().decode()
    assert err.startswith("ssu_scan") and "strides" in err


@pytest.mark.parametrize("batch,dim,G,L,chunk,N,want", [
    (2, 1024, 1, 4096, 512, 32, "scan_t16_n16_w1_c4"),   # one block, more than 16 states: not the one-block rule
    (3, 1024, 1, 4096, 512, 64, "scan_t16_n16_pair_c8"),
    (2, 1024, 1, 4096, 512, 1, "scan_t16_n16"),
])
def test_scan_select_tile_states(ssu, batch, dim, G, L, chunk, N, want):
    """The one-block rule is for up to 16 states per channel (one wave)."""
    a = _scan_args(ssu, batch=batch, dim=dim, G=G, L=L, N=N)
    t = ssu.scan_select_tile(a, chunk)
    assert t >= 0 and ssu.scan_tiles()[t] == want


@pytest.mark.parametrize("batch,dim,G,L,chunk,bstride,want", [
    (1, 1024, 1, 4096, 512, None, "scan_t16_n16"),          # up to 1024 channels: direct
    (1, 1024, 1, 4096, 128, None, "scan_t4_n16"),
    (2, 1024, 1, 4096, 512, None, "scan_t16_n16"),          # a launch of one block: direct up to 8192 channels
    (2, 1024, 1, 4096, 256, None, "scan_t8_n16"),
    (4, 1024, 1, 4096, 128, None, "scan_t4_n16"),
    (8, 1024, 1, 4096, 512, None, "scan_t16_n16"),
    (9, 1024, 1, 4096, 512, None, "scan_t16_n16_pair_c8"),  # above 8192: paired
    (2, 1024, 1, 4096, 1024, None, "scan_t16_n16_w1_c4"),   # up to 2048: staged for spans up to 1024
    (2, 1024, 1, 4096, 2048, None, "scan_t16_n16"),         # direct for longer spans
    (2, 1024, 1, 4096, 0, None, "scan_t16_n16"),
    (2, 1026, 1, 4096, 1024, None, "scan_t16_n16"),         # 1026 is not in fours: direct
    (3, 700, 1, 4096, 1024, None, "scan_t16_n16_w1_c4"),    # 2100 channels above 2048, 700 not in eights
    (3, 1024, 1, 4096, 1024, None, "scan_t16_n16_pair_c8"), # above: paired
    (16, 1024, 1, 4096, 0, None, "scan_t16_n16_pair_c8"),
    (3, 1028, 1, 4096, 1024, None, "scan_t16_n16_w1_c4"),   # a group's channels in fours only: staged
    (3, 1026, 1, 4096, 1024, None, "scan_t16_n16"),         # not in fours either: direct
    (3, 1024, 2, 4096, 1024, None, "scan_t16_n16_pair_c8"), # 512 channels per group
    (3, 1032, 2, 4096, 1024, None, "scan_t16_n16_w1_c4"),   # 516 per group
    (16, 1024, 1, 4096, 256, None, "scan_t8_n16_pair_c8"),  # the segment follows the launch's span
    (16, 1024, 1, 4096, 128, None, "scan_t4_n16_pair_c8"),
    (16, 1024, 1, 4096, 100, None, "scan_t2_n16_pair_c8"),
    (1, 64, 1, 300, 0, None, "scan_t8_n16"),
    (1, 64, 1, 300, 5000, None, "scan_t8_n16"),             # a chunk longer than L spans L
    (16, 1024, 1, 4096, 1024, (1 << 30) // 64, "scan_t16_n16"),  # row offsets beyond 32 bits: direct
])
def test_scan_select_tile(ssu, batch, dim, G, L, chunk, bstride, want):
    """The configuration ssu_scan picks by default, as ssu_scan_select_tile
    reports it (host logic only)."""
    a = _scan_args(ssu, batch=batch, dim=dim, G=G, L=L)
    if bstride is not None:
        a.B.stride[2] = bstride
    t = ssu.scan_select_tile(a, chunk)
    assert t >= 0 and ssu.scan_tiles()[t] == want


def test_scan_select_tile_invalid(ssu):
    assert ssu._lib.ssu_scan_select_tile(None, 0) == -1
    for mutate in (lambda a: setattr(a, "dim", 0), lambda a: setattr(a, "ngroups", 3),
                   lambda a: setattr(a, "seqlen", -1), lambda a: setattr(a, "batch", -1),
                   lambda a: a.C.stride.__setitem__(2, -1)):
        a = _scan_args(ssu)
        mutate(a)
        assert ssu.scan_select_tile(a, 0) == -1
    assert ssu.scan_select_tile(_scan_args(ssu), -1) == -1


def test_scan_empty_is_a_noop(ssu):
    """batch 0, or a sequence of length 0, returns OK without any HIP call."""
    a = _scan_args(ssu, batch=0)
    assert _scan_call(ssu, a) == 0
    a = _scan_args(ssu, L=0)
    a.u.ptr = a.delta.ptr = a.B.ptr = a.C.ptr = a.out.ptr = None  # never read when L == 0
    assert _scan_call(ssu, a) == 0


def test_scan_binding_validates(ssu):
    import torch

    u = torch.zeros((1, 4, 8), dtype=torch.float16)
    B = torch.zeros((1, 1, 16, 8), dtype=torch.float16)
    A = torch.zeros((4, 16))
    st = torch.zeros((1, 4, 16))
    with pytest.raises(ValueError, match="on a GPU"):
        ssu.make_scan_args(u, u, A, B, B, st)
    with pytest.raises(ValueError, match="delta shape"):
        ssu.make_scan_args(u, u[:, :2], A, B, B, st)
    with pytest.raises(TypeError, match="u's dtype"):
        ssu.make_scan_args(u, u.bfloat16(), A, B, B, st)
    with pytest.raises(TypeError):
        ssu.make_scan_args(u.float(), u.float(), A, B.float(), B.float(), st)


def test_handle_released_after_module_globals_are_cleared(ssu):
    """At interpreter exit a module's globals may be cleared (set to None)
    before the last handles are collected; a handle must still release itself
    then (seen as an 'Exception ignored in Handle.__del__' message at exit)."""
    h = ssu.Handle(16, 64, 128)
    saved = ssu._lib
    try:
        ssu._lib = None  # what finalization does to the module's globals
        h.__del__()
    finally:
        ssu._lib = saved
    assert h._h is None
