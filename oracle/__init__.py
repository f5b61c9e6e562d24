"""CPU oracle for the Mamba2 decode-step selective_state_update.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package. It
shares no code with the GPU library.

This module marshals numpy arrays into the plain-C fp64 oracle in
``ssu_ref.c`` (see that file for the definition it computes and the passages it
follows). Arrays are passed with their own strides, so the packed xBC views and
the per-head broadcasts reach the oracle exactly as they are stored. Besides
the decode step it holds the state-block copy and the selective scan over a
sequence (prefill), with the fp16 conversions the scan's io needs.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build_oracle

_i32, _i64 = ctypes.c_int32, ctypes.c_int64
_vp = ctypes.c_void_p


class RefArgs(ctypes.Structure):
    _fields_ = [
        ("batch", _i32), ("nheads", _i32), ("headdim", _i32), ("dstate", _i32),
        ("ngroups", _i32), ("dt_softplus", _i32), ("nsteps", _i32), ("nthreads", _i32),
        ("pool_slots", _i64),
        ("state", _vp), ("st_slot", _i64), ("st_head", _i64), ("st_row", _i64),
        ("idx", _vp),
        ("x", _vp), ("x_t", _i64), ("x_b", _i64), ("x_h", _i64), ("x_p", _i64),
        ("B", _vp), ("B_t", _i64), ("B_b", _i64), ("B_g", _i64), ("B_n", _i64),
        ("C", _vp), ("C_t", _i64), ("C_b", _i64), ("C_g", _i64), ("C_n", _i64),
        ("dt", _vp), ("dt_t", _i64), ("dt_b", _i64), ("dt_h", _i64),
        ("dt_bias", _vp), ("dt_bias_h", _i64),
        ("A", _vp), ("A_h", _i64),
        ("D", _vp), ("D_h", _i64),
        ("out", _vp), ("out_t", _i64), ("out_b", _i64), ("out_h", _i64), ("out_p", _i64),
        ("state_ref", _vp), ("y_ref", _vp), ("tau_ref", _vp),
    ]


def _estrides(a: np.ndarray):
    """Element strides of a numpy array (byte strides / itemsize)."""
    out = []
    for s in a.strides:
        if s % a.itemsize:
            raise ValueError("stride not a multiple of the element size")
        out.append(s // a.itemsize)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


class RefBlockTensor(ctypes.Structure):
    _fields_ = [("base", _vp), ("block_stride", _i64), ("block_bytes", _i64), ("nblocks", _i64)]


class RefScanArgs(ctypes.Structure):
    _fields_ = [
        ("batch", _i32), ("dim", _i32), ("dstate", _i32), ("ngroups", _i32),
        ("delta_softplus", _i32), ("io_dtype", _i32), ("nthreads", _i32), ("reserved", _i32),
        ("seqlen", _i64),
        ("state", _vp), ("st_b", _i64), ("st_d", _i64),
        ("u", _vp), ("u_b", _i64), ("u_d", _i64), ("u_t", _i64),
        ("delta", _vp), ("dl_b", _i64), ("dl_d", _i64), ("dl_t", _i64),
        ("B", _vp), ("B_b", _i64), ("B_g", _i64), ("B_n", _i64), ("B_t", _i64),
        ("C", _vp), ("C_b", _i64), ("C_g", _i64), ("C_n", _i64), ("C_t", _i64),
        ("A", _vp), ("A_d", _i64), ("A_n", _i64),
        ("D", _vp), ("delta_bias", _vp),
        ("out", _vp), ("o_b", _i64), ("o_d", _i64), ("o_t", _i64),
        ("state_ref", _vp), ("err_ref", _vp), ("y_ref", _vp), ("tau_ref", _vp), ("rho_ref", _vp),
    ]


IO_DTYPES = {"bf16": 0, "f16": 1}


class Oracle:
    """Handle on one build of the oracle library (the default build, or any other
    path, which the tests use to load deliberately broken copies)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = LIB_PATH
            if not os.path.exists(path):
                build_oracle()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.ssu_ref_run.argtypes = [ctypes.POINTER(RefArgs)]
        lib.ssu_ref_run.restype = _i32
        lib.ssu_ref_softplus.argtypes = [ctypes.c_double]
        lib.ssu_ref_softplus.restype = ctypes.c_double
        lib.ssu_ref_discretize.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, _i32,
                                           ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        lib.ssu_ref_discretize.restype = None
        lib.ssu_ref_bf16_rne.argtypes = [ctypes.c_float]
        lib.ssu_ref_bf16_rne.restype = ctypes.c_uint16
        lib.ssu_ref_copy_blocks.argtypes = [ctypes.POINTER(RefBlockTensor), _i32, ctypes.POINTER(_i32),
                                            ctypes.POINTER(_i32), _i32]
        lib.ssu_ref_copy_blocks.restype = _i32
        lib.ssu_ref_scan.argtypes = [ctypes.POINTER(RefScanArgs)]
        lib.ssu_ref_scan.restype = _i32
        lib.ssu_ref_f16_value.argtypes = [ctypes.c_uint16]
        lib.ssu_ref_f16_value.restype = ctypes.c_double
        lib.ssu_ref_f16_rne.argtypes = [ctypes.c_float]
        lib.ssu_ref_f16_rne.restype = ctypes.c_uint16
        lib.ssu_ref_max_threads.argtypes = []
        lib.ssu_ref_max_threads.restype = _i32
        self.lib = lib

    # -- scalar pieces -------------------------------------------------------
    def softplus(self, u: float) -> float:
        return self.lib.ssu_ref_softplus(float(u))

    def discretize(self, dt: float, dt_bias: float, A: float, softplus: bool = True):
        d, a = ctypes.c_double(), ctypes.c_double()
        self.lib.ssu_ref_discretize(float(dt), float(dt_bias), float(A), int(bool(softplus)),
                                    ctypes.byref(d), ctypes.byref(a))
        return d.value, a.value

    def bf16_rne(self, values) -> np.ndarray:
        v = np.asarray(values, dtype=np.float32).ravel()
        return np.array([self.lib.ssu_ref_bf16_rne(float(f)) for f in v], dtype=np.uint16)

    def f16_value(self, bits) -> np.ndarray:
        b = np.asarray(bits, dtype=np.uint16).ravel()
        return np.array([self.lib.ssu_ref_f16_value(int(v)) for v in b], dtype=np.float64)

    def f16_rne(self, values) -> np.ndarray:
        v = np.asarray(values, dtype=np.float32).ravel()
        return np.array([self.lib.ssu_ref_f16_rne(float(f)) for f in v], dtype=np.uint16)

    def max_threads(self) -> int:
        return int(self.lib.ssu_ref_max_threads())

    # -- block copy ------------------------------------------------------------
    def copy_blocks(self, tensors, src, dst):
        """Copy block src[r] to block dst[r] of every tensor in place.

        ``tensors``: numpy arrays whose axis 0 indexes blocks (a block is one
        ``arr[i]``, contiguous); src, dst: int32 [nreqs]."""
        src = np.ascontiguousarray(src, dtype=np.int32)
        dst = np.ascontiguousarray(dst, dtype=np.int32)
        if src.shape != dst.shape or src.ndim != 1:
            raise ValueError("src and dst must be int32 [nreqs]")
        descs = (RefBlockTensor * max(1, len(tensors)))()
        for k, arr in enumerate(tensors):
            if not arr.flags.writeable or not arr[0].flags.c_contiguous:
                raise ValueError("each tensor must be writeable with contiguous blocks")
            descs[k].base = arr.ctypes.data
            descs[k].block_stride = arr.strides[0]
            descs[k].block_bytes = arr[0].nbytes
            descs[k].nblocks = arr.shape[0]
        i32p = ctypes.POINTER(_i32)
        rc = self.lib.ssu_ref_copy_blocks(descs, len(tensors), src.ctypes.data_as(i32p),
                                          dst.ctypes.data_as(i32p), len(src))
        if rc != 0:
            raise ValueError({1: "bad argument", 2: "null pointer", 3: "overlapping destinations"}.get(rc, rc))

    # -- the step ------------------------------------------------------------
    def run(self, pool, idx, x, B, C, dt, A, dt_bias=None, D=None, dt_softplus=True,
            want_state=True, want_y=True, nthreads=0, out=None):
        """Advance ``pool`` (float32 numpy array [slots, H, P, N], updated in place)
        by one token (x [bs,H,P], B/C [bs,G,N], dt [bs,H]) or by K tokens
        (x [K,bs,H,P], B/C [K,bs,G,N], dt [K,bs,H]).

        Returns a dict: ``out`` (uint16 bf16 bits, shaped like x), ``y`` and
        ``tau`` (fp64, shaped like x) and ``state`` (fp64 [bs,H,P,N], S' after
        the last token) when requested.
        """
        single = x.ndim == 3
        if single:
            x, B, C, dt = x[None], B[None], C[None], dt[None]
        K, bs, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        if pool.dtype != np.float32 or pool.ndim != 4 or pool.shape[1:] != (H, P, N):
            raise ValueError(f"pool must be float32 [slots,{H},{P},{N}], got {pool.dtype} {pool.shape}")
        if pool.strides[3] != 4:
            raise ValueError("pool's dstate axis must be contiguous")
        if not pool.flags.writeable:
            raise ValueError("pool must be writeable")
        for name, arr, shp in (("B", B, (K, bs, G, N)), ("C", C, (K, bs, G, N)), ("dt", dt, (K, bs, H))):
            if arr.shape != shp:
                raise ValueError(f"{name} shape {arr.shape} != {shp}")
        for name, arr in (("x", x), ("B", B), ("C", C), ("dt", dt)):
            if arr.dtype != np.uint16:
                raise ValueError(f"{name} must hold bf16 bits (uint16)")
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        if idx.shape != (bs,):
            raise ValueError("idx must be [bs]")
        A = np.ascontiguousarray(A, dtype=np.float32)
        dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
        D = None if D is None else np.ascontiguousarray(D, dtype=np.float32)
        for name, arr in (("A", A), ("dt_bias", dt_bias), ("D", D)):
            if arr is not None and arr.shape != (H,):
                raise ValueError(f"{name} must be [H]")
        if out is None:
            out = np.zeros((K, bs, H, P), dtype=np.uint16)
        elif single:
            out = out[None]
        y = np.full((K, bs, H, P), np.nan) if want_y else None
        tau = np.full((K, bs, H, P), np.nan) if want_y else None
        state = np.full((bs, H, P, N), np.nan) if want_state else None

        a = RefArgs()
        a.batch, a.nheads, a.headdim, a.dstate, a.ngroups = bs, H, P, N, G
        a.dt_softplus, a.nsteps, a.nthreads = int(bool(dt_softplus)), K, int(nthreads)
        a.pool_slots = pool.shape[0]
        a.state = _ptr(pool)
        a.st_slot, a.st_head, a.st_row, _ = _estrides(pool)
        a.idx = _ptr(idx)
        a.x = _ptr(x)
        a.x_t, a.x_b, a.x_h, a.x_p = _estrides(x)
        a.B = _ptr(B)
        a.B_t, a.B_b, a.B_g, a.B_n = _estrides(B)
        a.C = _ptr(C)
        a.C_t, a.C_b, a.C_g, a.C_n = _estrides(C)
        a.dt = _ptr(dt)
        a.dt_t, a.dt_b, a.dt_h = _estrides(dt)
        a.dt_bias, a.dt_bias_h = _ptr(dt_bias), 1
        a.A, a.A_h = _ptr(A), 1
        a.D, a.D_h = _ptr(D), 1
        a.out = _ptr(out)
        a.out_t, a.out_b, a.out_h, a.out_p = _estrides(out)
        a.state_ref, a.y_ref, a.tau_ref = _ptr(state), _ptr(y), _ptr(tau)
        # keep every array alive across the call
        keep = (pool, idx, x, B, C, dt, A, dt_bias, D, out, y, tau, state)
        rc = self.lib.ssu_ref_run(ctypes.byref(a))
        del keep
        if rc != 0:
            raise ValueError({1: "bad shape", 2: "null pointer", 3: "duplicate slot index"}.get(rc, rc))
        res = {"out": out[0] if single else out}
        if want_y:
            res["y"] = y[0] if single else y
            res["tau"] = tau[0] if single else tau
        if want_state:
            res["state"] = state
        return res

    # -- selective scan over a sequence -------------------------------------
    def scan(self, state, u, delta, A, B, C, D=None, delta_bias=None, delta_softplus=True, io="f16",
              want_ref=True, nthreads=0, out=None):
        """Selective scan over a sequence (see ssu_ref.c), ``state`` updated in place.

        state: float32 [batch, dim, dstate] (dstate contiguous); u, delta: uint16
        bits [batch, dim, L]; B, C: uint16 bits [batch, G, dstate, L]; A: float32
        [dim, dstate]; D, delta_bias: float32 [dim] or None; io: "f16" or "bf16".

        Returns a dict: ``out`` (uint16 bits [batch, dim, L]) and, with want_ref,
        ``y``, ``tau``, ``rho`` (fp64 [batch, dim, L]), ``state`` and ``err``
        (fp64 [batch, dim, dstate]).
        """
        bs, dim, L = u.shape
        G, N = B.shape[1], B.shape[2]
        if state.dtype != np.float32 or state.shape != (bs, dim, N) or state.strides[2] != 4:
            raise ValueError(f"state must be float32 [{bs},{dim},{N}] with dstate contiguous")
        if not state.flags.writeable:
            raise ValueError("state must be writeable")
        for name, arr, shp in (("delta", delta, (bs, dim, L)), ("B", B, (bs, G, N, L)), ("C", C, (bs, G, N, L))):
            if arr.shape != shp:
                raise ValueError(f"{name} shape {arr.shape} != {shp}")
        for name, arr in (("u", u), ("delta", delta), ("B", B), ("C", C)):
            if arr.dtype != np.uint16:
                raise ValueError(f"{name} must hold {io} bits (uint16)")
        A = np.asarray(A, dtype=np.float32)
        if A.shape != (dim, N):
            raise ValueError("A must be [dim, dstate]")
        D = None if D is None else np.ascontiguousarray(D, dtype=np.float32)
        delta_bias = None if delta_bias is None else np.ascontiguousarray(delta_bias, dtype=np.float32)
        for name, arr in (("D", D), ("delta_bias", delta_bias)):
            if arr is not None and arr.shape != (dim,):
                raise ValueError(f"{name} must be [dim]")
        if out is None:
            out = np.zeros((bs, dim, L), dtype=np.uint16)
        refs = {}
        if want_ref:
            for k, shp in (("y", (bs, dim, L)), ("tau", (bs, dim, L)), ("rho", (bs, dim, L)),
                           ("state", (bs, dim, N)), ("err", (bs, dim, N))):
                refs[k] = np.full(shp, np.nan)
        a = RefScanArgs()
        a.batch, a.dim, a.dstate, a.ngroups = bs, dim, N, G
        a.delta_softplus, a.io_dtype, a.nthreads = int(bool(delta_softplus)), IO_DTYPES[io], int(nthreads)
        a.seqlen = L
        a.state = _ptr(state)
        a.st_b, a.st_d, _ = _estrides(state)
        a.u = _ptr(u)
        a.u_b, a.u_d, a.u_t = _estrides(u)
        a.delta = _ptr(delta)
        a.dl_b, a.dl_d, a.dl_t = _estrides(delta)
        a.B = _ptr(B)
        a.B_b, a.B_g, a.B_n, a.B_t = _estrides(B)
        a.C = _ptr(C)
        a.C_b, a.C_g, a.C_n, a.C_t = _estrides(C)
        a.A = _ptr(A)
        a.A_d, a.A_n = _estrides(A)
        a.D, a.delta_bias = _ptr(D), _ptr(delta_bias)
        a.out = _ptr(out)
        a.o_b, a.o_d, a.o_t = _estrides(out)
        a.state_ref, a.err_ref = _ptr(refs.get("state")), _ptr(refs.get("err"))
        a.y_ref, a.tau_ref, a.rho_ref = _ptr(refs.get("y")), _ptr(refs.get("tau")), _ptr(refs.get("rho"))
        keep = (state, u, delta, A, B, C, D, delta_bias, out, refs)
        rc = self.lib.ssu_ref_scan(ctypes.byref(a))
        del keep
        if rc != 0:
            raise ValueError({1: "bad shape", 2: "null pointer"}.get(rc, rc))
        return {"out": out, **refs}



_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from oracle/ssu_ref.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
