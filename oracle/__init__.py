"""Oracle for the dual-weight GLU projection and the grouped GEMV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``glu_mlp_gemv_amd``; neither imports the other.

The arithmetic lives in ``glu_oracle.c`` (fp64 dot products, bf16 rounding of
gate and up, fp32 silu rounded to bf16, bf16 product; its header states the
definition and the passages it follows).  This module is a ctypes face over it
that takes and returns numpy ``uint16`` arrays holding bf16 bit patterns.  The
backward (gradients of hidden and of both weights) is ``oracle.backward``, in
numpy over this module's forward sums.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import NamedTuple, Optional

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _bind(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    lib.glu_oracle_dual_gemv.argtypes = [
        _u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _f64p, _f64p, _f64p, _f64p, ctypes.c_int,
    ]
    lib.glu_oracle_dual_gemv.restype = ctypes.c_int
    lib.glu_oracle_dual_gemv_sampled.argtypes = [
        _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64p, _i64p, _i64,
        _u16p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int,
    ]
    lib.glu_oracle_dual_gemv_sampled.restype = ctypes.c_int
    lib.glu_oracle_epilogue.argtypes = [_u16p, _u16p, _u16p, _i64]
    lib.glu_oracle_epilogue.restype = ctypes.c_int
    lib.glu_oracle_silu_bf16.argtypes = [_u16p, _u16p, _i64]
    lib.glu_oracle_silu_bf16.restype = ctypes.c_int
    lib.glu_oracle_round_bf16.argtypes = [_f64p, _u16p, _i64]
    lib.glu_oracle_round_bf16.restype = ctypes.c_int
    lib.glu_oracle_linear.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, _f64p, _f64p, ctypes.c_int]
    lib.glu_oracle_linear.restype = ctypes.c_int
    lib.glu_oracle_max_threads.argtypes = []
    lib.glu_oracle_max_threads.restype = ctypes.c_int
    return lib


_DEFAULT: Optional[ctypes.CDLL] = None
_ACTIVE: Optional[ctypes.CDLL] = None


def _load() -> ctypes.CDLL:
    global _DEFAULT
    if _ACTIVE is not None:
        return _ACTIVE
    if _DEFAULT is None:
        # a sanitized build of the same source (glu_mlp_gemv_amd/sanitize.py) may be named here
        alt = os.environ.get("GLU_ORACLE_LIBRARY")
        if alt:
            _DEFAULT = _bind(alt)
            return _DEFAULT
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        _DEFAULT = _bind(_build.LIBRARY)
    return _DEFAULT


@contextlib.contextmanager
def using_library(path: str):
    """Route every call in this module to another build of the oracle source.

    Used only by the tests that compile a copy of the oracle with one planted
    mistake and check that the pins reject it.
    """
    global _ACTIVE
    prev = _ACTIVE
    _ACTIVE = _bind(path)
    try:
        yield
    finally:
        _ACTIVE = prev


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {a.dtype}")
    return a


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return ctypes.cast(None, ctype)
    return a.ctypes.data_as(ctype)


class DualGemvResult(NamedTuple):
    out: np.ndarray        # uint16 [M,N] bf16 bits
    gate_pre: np.ndarray   # fp64 [M,N]  G = h . Wg[j]
    up_pre: np.ndarray     # fp64 [M,N]  U = h . Wu[j]
    gate_abs: np.ndarray   # fp64 [M,N]  sum |h * Wg[j]|
    up_abs: np.ndarray     # fp64 [M,N]  sum |h * Wu[j]|


def dual_gemv(hidden: np.ndarray, gate_w: np.ndarray, up_w: np.ndarray,
              threads: int = 0, with_pre: bool = False):
    """out[m,j] of the GLU projection for bf16 bit arrays hidden [M,K], gate_w/up_w [N,K].

    With ``with_pre`` the fp64 pre-activations and absolute sums come back too
    (a :class:`DualGemvResult`); otherwise only the uint16 ``out`` array.
    """
    h = _u16(hidden)
    wg = _u16(gate_w)
    wu = _u16(up_w)
    if h.ndim != 2 or wg.ndim != 2 or wu.ndim != 2:
        raise ValueError("hidden, gate_w, up_w must be 2-D")
    M, K = h.shape
    N = wg.shape[0]
    if wg.shape != (N, K) or wu.shape != (N, K):
        raise ValueError(f"shape mismatch: hidden {h.shape}, gate_w {wg.shape}, up_w {wu.shape}")
    out = np.zeros((M, N), dtype=np.uint16)
    pre = [np.zeros((M, N), dtype=np.float64) for _ in range(4)] if with_pre else [None] * 4
    rc = _load().glu_oracle_dual_gemv(
        _ptr(h, _u16p), _ptr(wg, _u16p), _ptr(wu, _u16p), _ptr(out, _u16p),
        M, N, K, *(_ptr(p, _f64p) for p in pre), int(threads))
    if rc != 0:
        raise RuntimeError(f"glu_oracle_dual_gemv failed ({rc})")
    if with_pre:
        return DualGemvResult(out, *pre)
    return out


class LinearResult(NamedTuple):
    out: np.ndarray   # uint16 [M,N] bf16 bits
    pre: np.ndarray   # fp64 [M,N]  h . W[j]
    abs: np.ndarray   # fp64 [M,N]  sum |h * W[j]|


def linear(hidden: np.ndarray, w: np.ndarray, threads: int = 0, with_pre: bool = False):
    """One projection of a grouped GEMV: bf16(hidden @ w^T) for bf16 bit arrays hidden [M,K], w [N,K].

    With ``with_pre`` the fp64 dot products and absolute sums come back too (a
    :class:`LinearResult`); otherwise only the uint16 ``out`` array.
    """
    h = _u16(hidden)
    ww = _u16(w)
    if h.ndim != 2 or ww.ndim != 2 or ww.shape[1] != h.shape[1]:
        raise ValueError(f"shape mismatch: hidden {h.shape}, w {ww.shape}")
    M, K = h.shape
    N = ww.shape[0]
    out = np.zeros((M, N), dtype=np.uint16)
    pre = [np.zeros((M, N), dtype=np.float64) for _ in range(2)] if with_pre else [None, None]
    rc = _load().glu_oracle_linear(_ptr(h, _u16p), _ptr(ww, _u16p), _ptr(out, _u16p), M, N, K,
                                   *(_ptr(p, _f64p) for p in pre), int(threads))
    if rc != 0:
        raise RuntimeError(f"glu_oracle_linear failed ({rc})")
    if with_pre:
        return LinearResult(out, *pre)
    return out


def dual_gemv_sampled(hidden: np.ndarray, gate_w: np.ndarray, up_w: np.ndarray,
                      rows_m: np.ndarray, cols_j: np.ndarray, threads: int = 0) -> DualGemvResult:
    """The projection at listed (m, j) positions only; arrays indexed by list position."""
    h = _u16(hidden)
    wg = _u16(gate_w)
    wu = _u16(up_w)
    M, K = h.shape
    N = wg.shape[0]
    if wg.shape != (N, K) or wu.shape != (N, K):
        raise ValueError("shape mismatch")
    rm = np.ascontiguousarray(rows_m, dtype=np.int64)
    cj = np.ascontiguousarray(cols_j, dtype=np.int64)
    if rm.shape != cj.shape or rm.ndim != 1:
        raise ValueError("rows_m and cols_j must be 1-D of equal length")
    n = rm.shape[0]
    out = np.zeros(n, dtype=np.uint16)
    pre = [np.zeros(n, dtype=np.float64) for _ in range(4)]
    rc = _load().glu_oracle_dual_gemv_sampled(
        _ptr(h, _u16p), _ptr(wg, _u16p), _ptr(wu, _u16p), M, N, K,
        _ptr(rm, _i64p), _ptr(cj, _i64p), n, _ptr(out, _u16p),
        *(_ptr(p, _f64p) for p in pre), int(threads))
    if rc != 0:
        raise RuntimeError(f"glu_oracle_dual_gemv_sampled failed ({rc})")
    return DualGemvResult(out, *pre)


def epilogue(g_bits: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """Steps after the dots: bf16 silu of g, times u, rounded to bf16 (elementwise)."""
    g = _u16(g_bits).ravel()
    u = _u16(u_bits).ravel()
    if g.shape != u.shape:
        raise ValueError("g and u must have the same size")
    out = np.zeros_like(g)
    rc = _load().glu_oracle_epilogue(_ptr(g, _u16p), _ptr(u, _u16p), _ptr(out, _u16p), g.size)
    if rc != 0:
        raise RuntimeError("glu_oracle_epilogue failed")
    return out.reshape(np.shape(g_bits))


def silu_bf16(g_bits: np.ndarray) -> np.ndarray:
    """bf16 silu of bf16 inputs (fp32 evaluation, one rounding to bf16)."""
    g = _u16(g_bits).ravel()
    out = np.zeros_like(g)
    rc = _load().glu_oracle_silu_bf16(_ptr(g, _u16p), _ptr(out, _u16p), g.size)
    if rc != 0:
        raise RuntimeError("glu_oracle_silu_bf16 failed")
    return out.reshape(np.shape(g_bits))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to bf16 bit patterns, to nearest, ties to even."""
    a = np.ascontiguousarray(x, dtype=np.float64).ravel()
    out = np.zeros(a.shape, dtype=np.uint16)
    rc = _load().glu_oracle_round_bf16(_ptr(a, _f64p), _ptr(out, _u16p), a.size)
    if rc != 0:
        raise RuntimeError("glu_oracle_round_bf16 failed")
    return out.reshape(np.shape(x))


def max_threads() -> int:
    """OpenMP threads a parallel oracle call uses by default."""
    return int(_load().glu_oracle_max_threads())
