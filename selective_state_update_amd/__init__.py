"""selective_state_update_amd: the Mamba2 decode-step selective_state_update on
AMD Instinct MI355X (gfx950).

A thin ctypes binding over libssu (include/ssu.h). It checks tensor shapes,
dtypes and devices, turns torch tensors into (pointer, dtype tag, strides)
views, and calls ``ssu_update`` on the current HIP stream. All arithmetic runs
in the library's HIP kernel; nothing here computes, and there is no fallback:
if libssu.so is missing the import fails.

The operation follows the problem statement of sglang PR #41223 ("[Perf]
Mamba2 selective_state_update up to 2x faster on B200 via 8x1 launch config for
dstate 128", section "Kernel measurement"): an fp32 state pool [pool, H, P, N]
addressed by state_batch_indices, x [bs, H, P] and B/C [bs, G, N] in bf16 (they
may be views into one packed tensor), and dt, A, D, dt_bias broadcast
per head. Per request b and head h:

    delta = softplus(dt + dt_bias);  a = exp(A * delta)
    state[idx[b], h] = state[idx[b], h] * a + delta * outer(x[b, h], B[b, g])
    out[b, h] = state[idx[b], h] @ C[b, g] + D * x[b, h]      (bf16)
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "SSUError",
    "Handle",
    "selective_state_update",
    "TokensArgs",
    "copy_blocks",
    "copy_tiles",
    "ScanArgs",
    "make_scan_args",
    "selective_scan",
    "scan_launch",
    "scan_select_tile",
    "scan_tiles",
    "tile_fits",
    "tiles",
    "library_path",
    "abi_version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssu.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python selective_state_update_amd/build.py` "
        "(there is no fallback implementation)"
    )

# libssu must bind to the HIP runtime torch has loaded. torch ships its own
# libamdhip64 (soname libamdhip64.so.7) and its libraries ask for it by file
# name; if libssu were loaded first, it would bring in the system ROCm's
# runtime under that soname, torch would then load its own copy as well, and
# one of the two runtimes would see no device. Importing torch first makes
# libssu's libamdhip64.so.7 resolve to torch's copy.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(_LIB_PATH)

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

# ssu_status
SSU_OK = 0
STATUS_NAMES = {
    0: "SSU_OK",
    1: "SSU_ERR_INVALID_ARGUMENT",
    2: "SSU_ERR_UNSUPPORTED",
    3: "SSU_ERR_MISALIGNED",
    4: "SSU_ERR_HIP",
    5: "SSU_ERR_NO_MEMORY",
    6: "SSU_ERR_BAD_INDEX",
}
# ssu_dtype
SSU_F32, SSU_BF16, SSU_I32, SSU_I64, SSU_F16 = 0, 1, 2, 3, 4


class Config(ctypes.Structure):
    _fields_ = [("nheads", _i32), ("headdim", _i32), ("dstate", _i32), ("ngroups", _i32),
                ("dt_softplus", _i32), ("tile", _i32), ("device", _i32), ("reserved", _i32)]


class View(ctypes.Structure):
    _fields_ = [("ptr", _vp), ("dtype", _i32), ("reserved", _i32), ("stride", _i64 * 4)]


class Args(ctypes.Structure):
    _fields_ = [("batch", _i32), ("reserved", _i32), ("pool_slots", _i64),
                ("state", View), ("idx", View), ("x", View), ("B", View), ("C", View),
                ("dt", View), ("dt_bias", View), ("A", View), ("D", View), ("out", View)]


class TokensArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("ntokens", _i32), ("pool_slots", _i64),
                ("state", View), ("idx", View), ("x", View), ("B", View), ("C", View),
                ("dt", View), ("dt_bias", View), ("A", View), ("D", View), ("out", View)]


class BlockTensor(ctypes.Structure):
    _fields_ = [("base", _vp), ("block_stride", _i64), ("block_bytes", _i64), ("nblocks", _i64)]


class ScanArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("dim", _i32), ("dstate", _i32), ("ngroups", _i32), ("seqlen", _i64),
                ("delta_softplus", _i32), ("reserved", _i32),
                ("state", View), ("u", View), ("delta", View), ("B", View), ("C", View), ("A", View),
                ("D", View), ("delta_bias", View), ("out", View)]


class TileDesc(ctypes.Structure):
    _fields_ = [("dstate", _i32), ("rows_per_wave", _i32), ("waves", _i32), ("rows_per_group", _i32),
                ("nontemporal", _i32), ("xcd_remap", _i32), ("groups_per_cu", _i32), ("name", ctypes.c_char * 48)]


_lib.ssu_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_vp)]
_lib.ssu_create.restype = _i32
_lib.ssu_update.argtypes = [_vp, ctypes.POINTER(Args), _vp]
_lib.ssu_update.restype = _i32
_lib.ssu_update_tokens.argtypes = [_vp, ctypes.POINTER(TokensArgs), _vp]
_lib.ssu_update_tokens.restype = _i32
_lib.ssu_destroy.argtypes = [_vp]
_lib.ssu_destroy.restype = None
_lib.ssu_check_indices.argtypes = [ctypes.POINTER(Args), _vp]
_lib.ssu_check_indices.restype = _i32
_lib.ssu_select_tile.argtypes = [_vp, _i32]
_lib.ssu_select_tile.restype = _i32
_lib.ssu_select_tile_tokens.argtypes = [_vp, _i32, _i32]
_lib.ssu_select_tile_tokens.restype = _i32
_lib.ssu_tile_count.argtypes = []
_lib.ssu_tile_count.restype = _i32
_lib.ssu_tile_info.argtypes = [_i32, ctypes.POINTER(TileDesc)]
_lib.ssu_tile_info.restype = _i32
_lib.ssu_status_string.argtypes = [_i32]
_lib.ssu_status_string.restype = ctypes.c_char_p
_lib.ssu_last_error.argtypes = []
_lib.ssu_last_error.restype = ctypes.c_char_p
_lib.ssu_copy_blocks.argtypes = [ctypes.POINTER(BlockTensor), _i32, _vp, _vp, _i32, _i32, _vp]
_lib.ssu_copy_blocks.restype = _i32
_lib.ssu_copy_tile_count.argtypes = []
_lib.ssu_copy_tile_count.restype = _i32
_lib.ssu_copy_tile_name.argtypes = [_i32]
_lib.ssu_copy_tile_name.restype = ctypes.c_char_p
_lib.ssu_scan.argtypes = [ctypes.POINTER(ScanArgs), _i64, _i32, _vp]
_lib.ssu_scan.restype = _i32
_lib.ssu_scan_tile_count.argtypes = []
_lib.ssu_scan_tile_count.restype = _i32
_lib.ssu_scan_tile_name.argtypes = [_i32]
_lib.ssu_scan_tile_name.restype = ctypes.c_char_p
_lib.ssu_scan_select_tile.argtypes = [ctypes.POINTER(ScanArgs), _i64]
_lib.ssu_scan_select_tile.restype = _i32
_lib.ssu_abi_version.argtypes = []
_lib.ssu_abi_version.restype = _i32


class SSUError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.ssu_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def abi_version() -> int:
    return int(_lib.ssu_abi_version())


def tiles():
    """All compiled launch configurations, as dicts (index = tile id)."""
    out = []
    for i in range(_lib.ssu_tile_count()):
        d = TileDesc()
        st = _lib.ssu_tile_info(i, ctypes.byref(d))
        if st != SSU_OK:
            raise SSUError(st, "ssu_tile_info")
        out.append(dict(id=i, dstate=d.dstate, rows_per_wave=d.rows_per_wave, waves=d.waves,
                        rows_per_group=d.rows_per_group, nontemporal=d.nontemporal,
                        xcd_remap=d.xcd_remap, groups_per_cu=d.groups_per_cu, name=d.name.decode()))
    return out


def tile_fits(t, nheads: int, headdim: int) -> bool:
    """Whether launch configuration `t` (a dict from tiles()) serves H heads of
    headdim P: its rows per group divide P, or each of its waves covers one
    whole head and its waves split the heads evenly (the library's rule)."""
    rg, rw = t["rows_per_group"], t["rows_per_wave"]
    if headdim % rg == 0:
        return True
    return rw == headdim and rg % headdim == 0 and nheads % (rg // headdim) == 0


def _torch():
    import torch

    return torch


def _dtype_tag(t, allowed, name):
    torch = _torch()
    tags = {torch.float32: SSU_F32, torch.bfloat16: SSU_BF16, torch.int32: SSU_I32, torch.int64: SSU_I64,
            torch.float16: SSU_F16}
    tag = tags.get(t.dtype)
    if tag not in allowed:
        raise TypeError(f"{name}: dtype {t.dtype} not supported here")
    return tag


def _view(t, strides, tag) -> View:
    v = View()
    v.ptr = t.data_ptr()
    v.dtype = tag
    v.reserved = 0
    for i, s in enumerate(strides):
        v.stride[i] = int(s)
    return v


def _stream_of(stream, device):
    """hipStream_t for ``stream``: a torch stream, a raw handle, or None for
    torch's current stream on ``device`` (the operands' device)."""
    if stream is None:
        return _torch().cuda.current_stream(device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _null_view() -> View:
    v = View()
    v.ptr = None
    return v


class Handle:
    """A libssu handle for one (H, P, N, G, softplus) shape.

    ``tile`` = -1 uses the library's launch table; a tile id forces one launch
    configuration (see ``tiles()``); the SSU_TILE environment variable does the
    same for handles created with -1.
    """

    def __init__(self, nheads: int, headdim: int, dstate: int, ngroups: int = 1,
                 dt_softplus: bool = True, tile: int = -1, device: int = -1):
        cfg = Config(nheads, headdim, dstate, ngroups, int(bool(dt_softplus)), tile, device, 0)
        h = _vp()
        st = _lib.ssu_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != SSU_OK:
            raise SSUError(st, "ssu_create")
        self._h = h
        self.nheads, self.headdim, self.dstate, self.ngroups = nheads, headdim, dstate, ngroups
        self.dt_softplus = bool(dt_softplus)
        self.tile = tile

    # bound when the class is defined: at interpreter exit the module's
    # globals may already be cleared when the last handles are collected
    def __del__(self, _destroy=_lib.ssu_destroy):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _destroy(h)
            self._h = None

    def selected_tile(self, batch: int, ntokens: int = 1) -> int:
        if ntokens > 1:
            return int(_lib.ssu_select_tile_tokens(self._h, int(batch), int(ntokens)))
        return int(_lib.ssu_select_tile(self._h, int(batch)))

    # -- argument marshalling -------------------------------------------------
    def make_args(self, state, state_batch_indices, x, B, C, dt, A, D=None, dt_bias=None, out=None):
        """Check shapes/devices and build the ssu_args struct (no device work)."""
        H, P, N, G = self.nheads, self.headdim, self.dstate, self.ngroups
        if x.dim() != 3 or tuple(x.shape[1:]) != (H, P):
            raise ValueError(f"x must be [batch, {H}, {P}], got {tuple(x.shape)}")
        bs = x.shape[0]
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, P, N):
            raise ValueError(f"state must be [pool, {H}, {P}, {N}], got {tuple(state.shape)}")
        for name, t in (("B", B), ("C", C)):
            if tuple(t.shape) != (bs, G, N):
                raise ValueError(f"{name} must be [{bs}, {G}, {N}], got {tuple(t.shape)}")
        if state_batch_indices is None or tuple(state_batch_indices.shape) != (bs,):
            raise ValueError(f"state_batch_indices must be [{bs}]")
        if out is None:
            raise ValueError("out is required")
        if tuple(out.shape) != (bs, H, P):
            raise ValueError(f"out must be [{bs}, {H}, {P}], got {tuple(out.shape)}")
        dev = state.device
        if dev.type != "cuda":
            raise ValueError("state must be on a GPU")
        for name, t in (("state_batch_indices", state_batch_indices), ("x", x), ("B", B), ("C", C),
                        ("dt", dt), ("A", A), ("D", D), ("dt_bias", dt_bias), ("out", out)):
            if t is not None and t.device != dev:
                raise ValueError(f"{name} is on {t.device}, state on {dev}")

        # dt: [bs, H] or [bs, H, P] with stride 0 over P
        if dt.dim() == 2 and tuple(dt.shape) == (bs, H):
            dt_s = (dt.stride(0), dt.stride(1), 0)
        elif dt.dim() == 3 and tuple(dt.shape) == (bs, H, P):
            dt_s = tuple(dt.stride())
        else:
            raise ValueError(f"dt must be [{bs}, {H}] or [{bs}, {H}, {P}], got {tuple(dt.shape)}")

        def per_head(t, name, full):
            if t is None:
                return None
            if t.dim() == 1 and t.shape[0] == H:
                return (t.stride(0),) + (0,) * (len(full) - 1)
            if tuple(t.shape) == full:
                return tuple(t.stride())
            raise ValueError(f"{name} must be [{H}] or {list(full)}, got {tuple(t.shape)}")

        A_s = per_head(A, "A", (H, P, N))
        D_s = per_head(D, "D", (H, P))
        bias_s = per_head(dt_bias, "dt_bias", (H, P))

        a = Args()
        a.batch = bs
        a.reserved = 0
        a.pool_slots = state.shape[0]
        a.state = _view(state, state.stride(), _dtype_tag(state, (SSU_F32,), "state"))
        a.idx = _view(state_batch_indices, state_batch_indices.stride(),
                      _dtype_tag(state_batch_indices, (SSU_I32, SSU_I64), "state_batch_indices"))
        a.x = _view(x, x.stride(), _dtype_tag(x, (SSU_BF16,), "x"))
        a.B = _view(B, B.stride(), _dtype_tag(B, (SSU_BF16,), "B"))
        a.C = _view(C, C.stride(), _dtype_tag(C, (SSU_BF16,), "C"))
        a.dt = _view(dt, dt_s, _dtype_tag(dt, (SSU_BF16,), "dt"))
        a.A = _view(A, A_s, _dtype_tag(A, (SSU_F32,), "A"))
        a.D = _view(D, D_s, _dtype_tag(D, (SSU_F32,), "D")) if D is not None else _null_view()
        a.dt_bias = (_view(dt_bias, bias_s, _dtype_tag(dt_bias, (SSU_F32,), "dt_bias"))
                     if dt_bias is not None else _null_view())
        a.out = _view(out, out.stride(), _dtype_tag(out, (SSU_BF16,), "out"))
        return a

    def make_tokens_args(self, state, state_batch_indices, x, B, C, dt, A, D=None, dt_bias=None, out=None):
        """As make_args, for several tokens per request: x [bs, T, H, P],
        B/C [bs, T, G, N], dt [bs, T, H] (or [bs, T, H, P] with stride 0 over P),
        out [bs, T, H, P]."""
        H, P, N, G = self.nheads, self.headdim, self.dstate, self.ngroups
        if x.dim() != 4 or tuple(x.shape[2:]) != (H, P):
            raise ValueError(f"x must be [batch, tokens, {H}, {P}], got {tuple(x.shape)}")
        bs, T = x.shape[0], x.shape[1]
        if T < 1:
            raise ValueError("need at least one token")
        for name, t in (("B", B), ("C", C)):
            if tuple(t.shape) != (bs, T, G, N):
                raise ValueError(f"{name} must be [{bs}, {T}, {G}, {N}], got {tuple(t.shape)}")
        if out is None or tuple(out.shape) != (bs, T, H, P):
            raise ValueError(f"out must be [{bs}, {T}, {H}, {P}]")
        if dt.dim() == 3 and tuple(dt.shape) == (bs, T, H):
            dt_s = (dt.stride(0), dt.stride(1), dt.stride(2), 0)
        elif dt.dim() == 4 and tuple(dt.shape) == (bs, T, H, P):
            dt_s = tuple(dt.stride())
        else:
            raise ValueError(f"dt must be [{bs}, {T}, {H}] or [{bs}, {T}, {H}, {P}], got {tuple(dt.shape)}")
        # token 0's views go through the one-token checks (shapes, devices, dtypes)
        one = self.make_args(state, state_batch_indices, x[:, 0], B[:, 0], C[:, 0], dt[:, 0], A, D, dt_bias,
                             out[:, 0])
        a = TokensArgs()
        a.batch, a.ntokens, a.pool_slots = bs, T, one.pool_slots
        a.state, a.idx, a.A, a.D, a.dt_bias = one.state, one.idx, one.A, one.D, one.dt_bias
        a.x = _view(x, x.stride(), SSU_BF16)
        a.B = _view(B, B.stride(), SSU_BF16)
        a.C = _view(C, C.stride(), SSU_BF16)
        a.dt = _view(dt, dt_s, SSU_BF16)
        a.out = _view(out, out.stride(), SSU_BF16)
        return a

    def launch(self, args, stream=None, device=None):
        """Enqueue ssu_update (Args) or ssu_update_tokens (TokensArgs) with
        prepared arguments on ``stream`` (torch stream, raw hipStream_t int, or
        None for torch's current stream on ``device``, by default the current
        device)."""
        stream = _stream_of(stream, device)
        if isinstance(args, TokensArgs):
            st = _lib.ssu_update_tokens(self._h, ctypes.byref(args), _vp(stream))
            where = "ssu_update_tokens"
        else:
            st = _lib.ssu_update(self._h, ctypes.byref(args), _vp(stream))
            where = "ssu_update"
        if st != SSU_OK:
            raise SSUError(st, where)

    def update_tokens(self, state, state_batch_indices, x, B, C, dt, A, D=None, dt_bias=None, out=None,
                      stream=None):
        """Advance ``state`` in place by x.shape[1] tokens per request in one
        launch; returns out [bs, T, H, P] (bf16), out[:, t] after token t."""
        if out is None:
            out = _torch().empty(x.shape, dtype=_torch().bfloat16, device=x.device)
        args = self.make_tokens_args(state, state_batch_indices, x, B, C, dt, A, D, dt_bias, out)
        self.launch(args, stream, state.device)
        return out

    def update(self, state, state_batch_indices, x, B, C, dt, A, D=None, dt_bias=None, out=None,
               stream=None, check_indices=False):
        """Advance ``state`` in place by one token and return ``out`` (bf16 [bs, H, P])."""
        if out is None:
            out = _torch().empty(x.shape, dtype=_torch().bfloat16, device=x.device)
        args = self.make_args(state, state_batch_indices, x, B, C, dt, A, D, dt_bias, out)
        if check_indices:
            st = _lib.ssu_check_indices(ctypes.byref(args), _vp(_stream_of(stream, state.device)))
            if st != SSU_OK:
                raise SSUError(st, "ssu_check_indices")
        self.launch(args, stream, state.device)
        return out


_handles: dict = {}
_handles_lock = threading.Lock()


def selective_state_update(state, x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
                           state_batch_indices=None, out=None, tile=-1):
    """Functional form: one decode step on ``state`` (updated in place); returns out.

    state [pool, H, P, N] fp32; x [bs, H, P] bf16; dt [bs, H] (or [bs, H, P] with
    stride 0 over P) bf16; A [H] (or [H, P, N] stride-0) fp32; B, C [bs, G, N]
    bf16; D, dt_bias [H] (or [H, P] stride-0) fp32 or None; state_batch_indices
    [bs] int32/int64.
    """
    H, P, N = state.shape[1], state.shape[2], state.shape[3]
    G = B.shape[1]
    key = (H, P, N, G, bool(dt_softplus), tile, state.device.index)
    with _handles_lock:
        h = _handles.get(key)
        if h is None:
            h = Handle(H, P, N, G, dt_softplus, tile, -1 if state.device.index is None else state.device.index)
            _handles[key] = h
    return h.update(state, state_batch_indices, x, B, C, dt, A, D, dt_bias, out)


def copy_tiles():
    """Names of the compiled block-copy configurations (index = tile id)."""
    return [_lib.ssu_copy_tile_name(i).decode() for i in range(_lib.ssu_copy_tile_count())]


def block_tensors(tensors):
    """ssu_block_tensor descriptors for torch tensors whose axis 0 indexes
    blocks (block i is ``t[i]``, which must be contiguous)."""
    descs = (BlockTensor * max(1, len(tensors)))()
    for k, t in enumerate(tensors):
        if t.dim() < 1:
            raise ValueError(f"tensor {k}: axis 0 must index blocks")
        if t.shape[0] > 0 and not t[0].is_contiguous():
            raise ValueError(f"tensor {k}: block t[i] must be contiguous")
        if t.device.type != "cuda":
            raise ValueError(f"tensor {k} must be on a GPU")
        descs[k].base = t.data_ptr()
        descs[k].block_stride = t.stride(0) * t.element_size()
        descs[k].block_bytes = t[0].numel() * t.element_size()
        descs[k].nblocks = t.shape[0]
    return descs


def copy_blocks(tensors, src_blocks, dst_blocks, tile=-1, stream=None, descs=None):
    """Copy block src_blocks[r] to block dst_blocks[r] of every tensor
    (ssu_copy_blocks). src_blocks, dst_blocks: int32 GPU tensors [nreqs].
    ``descs`` may pass prepared block_tensors(tensors) to skip rebuilding them."""
    torch = _torch()
    if src_blocks.dtype != torch.int32 or dst_blocks.dtype != torch.int32:
        raise TypeError("block ids must be int32")
    if src_blocks.shape != dst_blocks.shape or src_blocks.dim() != 1:
        raise ValueError("src_blocks and dst_blocks must be [nreqs]")
    if not (src_blocks.is_contiguous() and dst_blocks.is_contiguous()):
        raise ValueError("block ids must be contiguous")
    if src_blocks.device.type != "cuda" or dst_blocks.device != src_blocks.device:
        raise ValueError("block ids must be on the same GPU")
    if any(t.device != src_blocks.device for t in tensors):
        raise ValueError("state tensors must be on the block ids' GPU")
    if descs is None:
        descs = block_tensors(tensors)
    elif len(descs) < len(tensors):
        raise ValueError("descs has fewer entries than tensors")
    st = _lib.ssu_copy_blocks(descs, len(tensors), src_blocks.data_ptr(), dst_blocks.data_ptr(),
                              src_blocks.shape[0], tile, _vp(_stream_of(stream, src_blocks.device)))
    if st != SSU_OK:
        raise SSUError(st, "ssu_copy_blocks")


# --------------------------------------------------------------------------- #
# Selective scan over a sequence (prefill): ssu_scan
# --------------------------------------------------------------------------- #
def scan_tiles():
    """Names of the compiled scan configurations (index = tile id)."""
    return [_lib.ssu_scan_tile_name(i).decode() for i in range(_lib.ssu_scan_tile_count())]


def make_scan_args(u, delta, A, B, C, state, D=None, delta_bias=None, delta_softplus=True, out=None):
    """ScanArgs for ssu_scan from torch GPU tensors.

    u, delta: [batch, dim, L] float16 or bfloat16 (token axis contiguous);
    B, C: [batch, G, dstate, L] same dtype; A: [dim, dstate] float32;
    state: [batch, dim, dstate] float32 (dstate contiguous), read and written;
    D, delta_bias: [dim] float32 or None. out (optional): like u.
    Returns (ScanArgs, out); the tensors must stay alive while it is used."""
    torch = _torch()
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, L]")
    bs, dim, L = u.shape
    if B.dim() != 4 or B.shape[0] != bs or B.shape[3] != L:
        raise ValueError("B must be [batch, G, dstate, L]")
    G, N = B.shape[1], B.shape[2]
    for name, t, shp in (("delta", delta, (bs, dim, L)), ("C", C, (bs, G, N, L)), ("A", A, (dim, N)),
                         ("state", state, (bs, dim, N))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shp}")
    io = (SSU_F16, SSU_BF16)
    ut = _dtype_tag(u, io, "u")
    for name, t in (("delta", delta), ("B", B), ("C", C)):
        if _dtype_tag(t, io, name) != ut:
            raise TypeError(f"{name} must have u's dtype")
    if u.device.type != "cuda":
        raise ValueError("u must be on a GPU")
    if out is None:
        out = torch.empty((bs, dim, L), dtype=u.dtype, device=u.device)
    elif tuple(out.shape) != (bs, dim, L) or out.dtype != u.dtype:
        raise ValueError("out must be like u")
    for name, t in (("delta", delta), ("B", B), ("C", C), ("A", A), ("state", state), ("D", D),
                    ("delta_bias", delta_bias), ("out", out)):
        if t is not None and t.device != u.device:
            raise ValueError(f"{name} is on {t.device}, u on {u.device}")
    a = ScanArgs()
    a.batch, a.dim, a.dstate, a.ngroups, a.seqlen = bs, dim, N, G, L
    a.delta_softplus, a.reserved = int(bool(delta_softplus)), 0
    a.state = _view(state, state.stride(), _dtype_tag(state, (SSU_F32,), "state"))
    a.u = _view(u, u.stride(), ut)
    a.delta = _view(delta, delta.stride(), ut)
    a.B = _view(B, B.stride(), ut)
    a.C = _view(C, C.stride(), ut)
    a.A = _view(A, A.stride(), _dtype_tag(A, (SSU_F32,), "A"))
    for name, t in (("D", D), ("delta_bias", delta_bias)):
        if t is None:
            setattr(a, name, _null_view())
            continue
        if tuple(t.shape) != (dim,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [dim] tensor")
        setattr(a, name, _view(t, t.stride(), _dtype_tag(t, (SSU_F32,), name)))
    a.out = _view(out, out.stride(), ut)
    return a, out


def scan_select_tile(args, chunk=0):
    """Index of the configuration ssu_scan picks for prepared ScanArgs and
    ``chunk`` (see include/ssu.h, ssu_scan_select_tile); -1 for invalid sizes."""
    return int(_lib.ssu_scan_select_tile(ctypes.byref(args), int(chunk)))


def scan_launch(args, chunk=0, tile=-1, stream=None, device=None):
    """ssu_scan on prepared ScanArgs (for timing loops and graph capture);
    stream None: torch's current stream on ``device`` (default: the current
    device)."""
    st = _lib.ssu_scan(ctypes.byref(args), int(chunk), int(tile), _vp(_stream_of(stream, device)))
    if st != SSU_OK:
        raise SSUError(st, "ssu_scan")


def selective_scan(u, delta, A, B, C, state, D=None, delta_bias=None, delta_softplus=True, out=None,
                   chunk=0, tile=-1, stream=None):
    """Scan a sequence (see include/ssu.h, ssu_scan): ``state`` advances in place
    over all L tokens, in launches of ``chunk`` tokens (0: one launch).
    Returns out [batch, dim, L] in u's dtype."""
    args, out = make_scan_args(u, delta, A, B, C, state, D, delta_bias, delta_softplus, out)
    scan_launch(args, chunk, tile, stream, u.device)
    return out
