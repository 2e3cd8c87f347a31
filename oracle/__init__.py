"""Exact-attention oracle: fp64 CPU reference (ctypes wrapper over attn_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports it and shares no code with it.

The definitions it follows are documented in ``attn_oracle.c``: the dense
``softmax(scale * Q K^T [+ causal]) V`` of the FlashAttention pages, the
blockwise online (m, l, u) merge, and the textbook backward with recomputed
probabilities.  Arrays are numpy, laid out [B, H, N, d]; any real dtype is
upcast to float64 (exact for bf16 and fp32 values) before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def compile_source(src: str, out: str) -> str:
    """gcc an oracle source file into a shared library (fp64, OpenMP, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", tmp, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile attn_oracle.c into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    d = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    ci, cd, c64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
    dims = [ci] * 7 + [ci, cd]  # B Hq Hkv Nq Nk dk dv causal scale
    lib.oracle_fwd.argtypes = [d, d, d, d, d] + dims
    lib.oracle_fwd_bottom_right.argtypes = [d, d, d, d, d] + dims
    lib.oracle_fwd_rows.argtypes = [d, d, d, i64p, c64, d, d] + dims
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_fwd_blockmask.argtypes = [d, d, d, d, d, u8p, ci, ci, ci] + [ci] * 6 + [ci, cd]
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_fwd_varlen.argtypes = [d, d, d, d, d, i32p] + [ci] * 6 + [ci, cd]
    lib.oracle_fwd_blockwise.argtypes = [d, d, d, d, d] + dims + [ci, ci]
    lib.oracle_bwd.argtypes = [d] * 10 + dims
    lib.oracle_bwd_slices.argtypes = [d, d, d, d, i64p, c64, d, d, d] + dims
    lib.oracle_threads.argtypes = []
    for f in (lib.oracle_threads, lib.oracle_fwd, lib.oracle_fwd_bottom_right, lib.oracle_fwd_rows,
              lib.oracle_fwd_blockmask, lib.oracle_fwd_varlen,
              lib.oracle_fwd_blockwise, lib.oracle_bwd, lib.oracle_bwd_slices):
        f.restype = ci
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _lib = _bind(_LIB_PATH)
    return _lib


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: exact upcast on the CPU
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("oracle expects [B, H, N, d] arrays")
    B, Hq, Nq, dk = q.shape
    Bk, Hkv, Nk, dk2 = k.shape
    Bv, Hv, Nv, dv = v.shape
    if (Bk, dk2) != (B, dk) or (Bv, Hv, Nv) != (Bk, Hkv, Nk):
        raise ValueError("oracle: inconsistent q/k/v shapes")
    return B, Hq, Hkv, Nq, Nk, dk, dv


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what} failed with status {rc}")


def default_scale(dk: int) -> float:
    return 1.0 / np.sqrt(dk)


class Oracle:
    """The oracle's entry points bound to one compiled library."""

    def __init__(self, lib=None):
        self._lib = lib

    @property
    def lib(self):
        return self._lib if self._lib is not None else _load()

    def fwd(self, q, k, v, causal: bool = False, scale: float | None = None):
        """Dense forward. Returns (O [B,Hq,Nq,dv], LSE [B,Hq,Nq]) in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        scale = default_scale(dk) if scale is None else float(scale)
        o = np.empty((B, Hq, Nq, dv), np.float64)
        lse = np.empty((B, Hq, Nq), np.float64)
        _check(self.lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   B, Hq, Hkv, Nq, Nk, dk, dv, int(bool(causal)), scale),
               "oracle_fwd")
        return o, lse

    def fwd_bottom_right(self, q, k, v, causal: bool = False, scale: float | None = None):
        """Dense forward with the causal mask aligned bottom-right (query i of Nq
        sees keys j <= i + Nk - Nq). Returns (O, LSE) in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        scale = default_scale(dk) if scale is None else float(scale)
        o = np.empty((B, Hq, Nq, dv), np.float64)
        lse = np.empty((B, Hq, Nq), np.float64)
        _check(self.lib.oracle_fwd_bottom_right(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                B, Hq, Hkv, Nq, Nk, dk, dv, int(bool(causal)),
                                                scale), "oracle_fwd_bottom_right")
        return o, lse

    def fwd_blockmask(self, q, k, v, mask, bm: int, bn: int, causal: bool = False,
                      scale: float | None = None):
        """Block-sparse forward: query i of head h sees key j iff
        mask[h or 0][i // bm][j // bn] (and j <= i when causal).  mask is uint8
        [1 or Hq, ceil(N/bm), ceil(N/bn)]. Returns (O, LSE) in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        if Nq != Nk:
            raise ValueError("block-sparse forward is square: Nq == Nk")
        m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
        nbq, nbk = -(-Nq // bm), -(-Nk // bn)
        if m.ndim != 3 or m.shape[0] not in (1, Hq) or m.shape[1:] != (nbq, nbk):
            raise ValueError(f"mask must be [1 or {Hq}, {nbq}, {nbk}], got {m.shape}")
        scale = default_scale(dk) if scale is None else float(scale)
        o = np.empty((B, Hq, Nq, dv), np.float64)
        lse = np.empty((B, Hq, Nq), np.float64)
        mp = m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        _check(self.lib.oracle_fwd_blockmask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), mp,
                                             m.shape[0], int(bm), int(bn), B, Hq, Hkv, Nq, dk,
                                             dv, int(bool(causal)), scale),
               "oracle_fwd_blockmask")
        return o, lse

    def fwd_varlen(self, q, k, v, cu_seqlens, causal: bool = False, scale: float | None = None):
        """Packed variable-length forward: q [Hq, T, dk], k/v [Hkv, T, d], sequences
        at token offsets cu_seqlens (0 = cu[0] <= ... <= cu[-1] = T), each attending
        only within itself. Returns (O [Hq, T, dv], LSE [Hq, T]) in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
            raise ValueError("varlen tensors are [H, T, d]")
        _, Hq, Hkv, T, _, dk, dv = _shapes(q[None], k[None], v[None])
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        scale = default_scale(dk) if scale is None else float(scale)
        o = np.empty((Hq, T, dv), np.float64)
        lse = np.empty((Hq, T), np.float64)
        _check(self.lib.oracle_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                          cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                          len(cu) - 1, Hq, Hkv, T, dk, dv, int(bool(causal)),
                                          scale), "oracle_fwd_varlen")
        return o, lse

    def fwd_rows(self, q, k, v, rows, causal: bool = False, scale: float | None = None):
        """Dense forward of selected flat rows ((b*Hq+h)*Nq+i). Returns (O [n,dv], LSE [n])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        scale = default_scale(dk) if scale is None else float(scale)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.size
        o = np.empty((n, dv), np.float64)
        lse = np.empty((n,), np.float64)
        _check(self.lib.oracle_fwd_rows(
            _ptr(q), _ptr(k), _ptr(v), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            n, _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, dk, dv, int(bool(causal)), scale),
            "oracle_fwd_rows")
        return o, lse

    def fwd_blockwise(self, q, k, v, causal: bool = False, scale: float | None = None,
                      br: int = 1, bc: int = 1):
        """Blockwise forward with the online (m, l, u) merge; same outputs as fwd()."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        scale = default_scale(dk) if scale is None else float(scale)
        o = np.empty((B, Hq, Nq, dv), np.float64)
        lse = np.empty((B, Hq, Nq), np.float64)
        _check(self.lib.oracle_fwd_blockwise(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, dk, dv,
            int(bool(causal)), scale, int(br), int(bc)), "oracle_fwd_blockwise")
        return o, lse

    def bwd(self, q, k, v, dout, causal: bool = False, scale: float | None = None,
            with_stats: bool = False):
        """Textbook backward. Returns (dQ, dK, dV) [+ (LSE, O, D) if with_stats]."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        if dout.shape != (B, Hq, Nq, dv):
            raise ValueError("oracle: dout shape must match O")
        scale = default_scale(dk) if scale is None else float(scale)
        dq = np.empty_like(q)
        dkk = np.empty_like(k)
        dvv = np.empty_like(v)
        lse = np.empty((B, Hq, Nq)) if with_stats else None
        o = np.empty((B, Hq, Nq, dv)) if with_stats else None
        dsum = np.empty((B, Hq, Nq)) if with_stats else None
        _check(self.lib.oracle_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dkk), _ptr(dvv),
            _ptr(lse), _ptr(o), _ptr(dsum), B, Hq, Hkv, Nq, Nk, dk, dv,
            int(bool(causal)), scale), "oracle_bwd")
        if with_stats:
            return dq, dkk, dvv, lse, o, dsum
        return dq, dkk, dvv

    def bwd_slices(self, q, k, v, dout, slices, causal: bool = False,
                   scale: float | None = None):
        """Backward of whole (b, kv-group) slices, slices[t] = b*Hkv+g.

        Returns dQ [n, group, Nq, dk], dK [n, Nk, dk], dV [n, Nk, dv].
        """
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, Nq, Nk, dk, dv = _shapes(q, k, v)
        scale = default_scale(dk) if scale is None else float(scale)
        slices = np.ascontiguousarray(np.asarray(slices, dtype=np.int64))
        n = slices.size
        group = Hq // Hkv
        dq = np.empty((n, group, Nq, dk))
        dkk = np.empty((n, Nk, dk))
        dvv = np.empty((n, Nk, dv))
        _check(self.lib.oracle_bwd_slices(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
            slices.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n,
            _ptr(dq), _ptr(dkk), _ptr(dvv), B, Hq, Hkv, Nq, Nk, dk, dv,
            int(bool(causal)), scale), "oracle_bwd_slices")
        return dq, dkk, dvv

    def omp_threads(self) -> int:
        """Threads the oracle's OpenMP parallel loops use in this process."""
        return int(self.lib.oracle_threads())


def from_library(path: str) -> Oracle:
    """Bind the entry points of another build of attn_oracle.c (used by tests
    that plant mistakes in a copy of the source to show the pins catch them)."""
    return Oracle(_bind(path))


_default = Oracle()
fwd = _default.fwd
fwd_rows = _default.fwd_rows
fwd_bottom_right = _default.fwd_bottom_right
fwd_blockwise = _default.fwd_blockwise
fwd_blockmask = _default.fwd_blockmask
fwd_varlen = _default.fwd_varlen
bwd = _default.bwd
bwd_slices = _default.bwd_slices
omp_threads = _default.omp_threads
