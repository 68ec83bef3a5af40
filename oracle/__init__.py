"""CPU fp64 oracle for AllGather->GEMM and GEMM->ReduceScatter.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library under test never does,
and this package imports nothing from it.

Thin ctypes wrapper over liboracle.so (oracle.c).  Inputs are numpy uint16
arrays of bf16 bit patterns; outputs are float64.  Shapes:
    ag_gemm:  x [N, m, k], w [N, n, k]    -> y   [N, N*m, n]
    gemm_rs:  h [N, N*m, k], w [N, n, k]  -> out [N, m, n]
    allreduce: same inputs as gemm_rs     -> ar  [N*m, n]
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def load(path=None):
    """Load liboracle.so (building it first if it is absent)."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _bind(ctypes.CDLL(_build.LIB))
    return _LIB


def _bind(lib):
    u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    f64p_or_null = ctypes.c_void_p
    ci = ctypes.c_int
    lib.orc_threads.restype = ci
    lib.orc_threads.argtypes = []
    for name in ("orc_ag_gemm", "orc_gemm_rs"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [ci, ci, ci, ci, u16p, u16p, f64p, f64p_or_null]
    for name in ("orc_ag_gemm_rows", "orc_gemm_rs_rows"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [ci, ci, ci, ci, u16p, u16p, ci, i32p, i32p, f64p, f64p_or_null]
    lib.orc_allreduce.restype = None
    lib.orc_allreduce.argtypes = [ci, ci, ci, ci, u16p, u16p, f64p]
    lib.orc_gemm_rs_bf16_bucket_rows.restype = None
    lib.orc_gemm_rs_bf16_bucket_rows.argtypes = [ci, ci, ci, ci, u16p, u16p, ci, ci, i32p, i32p, f64p, f64p_or_null, f64p_or_null]
    lib.orc_round_bf16.restype = None
    lib.orc_round_bf16.argtypes = [f64p, u16p, ctypes.c_size_t]
    return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16), got %s" % a.dtype)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads(lib=None):
    return (lib or load()).orc_threads()


def ag_gemm(x, w, with_mag=False, lib=None):
    """Y_r = concat_r(X_r) . W_r^T for every rank r; returns y (and mag)."""
    lib = lib or load()
    x, w = _u16(x), _u16(w)
    N, m, k = x.shape
    Nw, n, kw = w.shape
    assert Nw == N and kw == k
    y = np.empty((N, N * m, n), np.float64)
    mag = np.empty_like(y) if with_mag else None
    lib.orc_ag_gemm(N, m, k, n, x, w, y, _ptr(mag))
    return (y, mag) if with_mag else y


def ag_gemm_rows(x, w, ranks, rows, with_mag=False, lib=None):
    """Rows rows[s] of Y_{ranks[s]} only; returns [len(rows), n] (and mag)."""
    lib = lib or load()
    x, w = _u16(x), _u16(w)
    N, m, k = x.shape
    n = w.shape[1]
    ranks = np.ascontiguousarray(ranks, np.int32)
    rows = np.ascontiguousarray(rows, np.int32)
    assert ranks.shape == rows.shape and ranks.ndim == 1
    assert ((0 <= ranks) & (ranks < N)).all() and ((0 <= rows) & (rows < N * m)).all()
    y = np.empty((len(rows), n), np.float64)
    mag = np.empty_like(y) if with_mag else None
    lib.orc_ag_gemm_rows(N, m, k, n, x, w, len(rows), ranks, rows, y, _ptr(mag))
    return (y, mag) if with_mag else y


def gemm_rs(h, w, with_mag=False, lib=None):
    """Out_q = sum_r (H_r . W_r^T)[q*m:(q+1)*m]; returns out (and mag)."""
    lib = lib or load()
    h, w = _u16(h), _u16(w)
    N, T, k = h.shape
    Nw, n, kw = w.shape
    assert Nw == N and kw == k and T % N == 0
    m = T // N
    out = np.empty((N, m, n), np.float64)
    mag = np.empty_like(out) if with_mag else None
    lib.orc_gemm_rs(N, m, k, n, h, w, out, _ptr(mag))
    return (out, mag) if with_mag else out


def gemm_rs_rows(h, w, owners, rows, with_mag=False, lib=None):
    """Rows rows[s] of Out_{owners[s]} only; returns [len(rows), n] (and mag)."""
    lib = lib or load()
    h, w = _u16(h), _u16(w)
    N, T, k = h.shape
    n = w.shape[1]
    m = T // N
    owners = np.ascontiguousarray(owners, np.int32)
    rows = np.ascontiguousarray(rows, np.int32)
    assert owners.shape == rows.shape and owners.ndim == 1
    assert ((0 <= owners) & (owners < N)).all() and ((0 <= rows) & (rows < m)).all()
    out = np.empty((len(rows), n), np.float64)
    mag = np.empty_like(out) if with_mag else None
    lib.orc_gemm_rs_rows(N, m, k, n, h, w, len(rows), owners, rows, out, _ptr(mag))
    return (out, mag) if with_mag else out


def gemm_rs_bf16_bucket_rows(h, w, owners, rows, dir="uni", with_mag=False, lib=None):
    """GEMM -> ReduceScatter with the circulating bucket rounded to bf16 after
    every addition (see oracle.c).  Returns out [len(rows), n] (unrounded
    final sums), and with with_mag also mag (sum |a*w|) and rmag (sum of
    |bucket| over every rounding)."""
    lib = lib or load()
    h, w = _u16(h), _u16(w)
    N, T, k = h.shape
    n = w.shape[1]
    m = T // N
    owners = np.ascontiguousarray(owners, np.int32)
    rows = np.ascontiguousarray(rows, np.int32)
    assert owners.shape == rows.shape and owners.ndim == 1
    assert ((0 <= owners) & (owners < N)).all() and ((0 <= rows) & (rows < m)).all()
    out = np.empty((len(rows), n), np.float64)
    mag = np.empty_like(out) if with_mag else None
    rmag = np.empty_like(out) if with_mag else None
    lib.orc_gemm_rs_bf16_bucket_rows(N, m, k, n, h, w, 1 if dir == "bi" else 0, len(rows), owners, rows, out,
                                     _ptr(mag), _ptr(rmag))
    return (out, mag, rmag) if with_mag else out


def gemm_rs_bf16_bucket(h, w, dir="uni", with_mag=False, lib=None):
    """Every output row of the bf16-bucket GEMM -> ReduceScatter: [N][m][n]."""
    N, T, _ = np.asarray(h).shape
    m, n = T // N, np.asarray(w).shape[1]
    owners = np.repeat(np.arange(N), m)
    rows = np.tile(np.arange(m), N)
    res = gemm_rs_bf16_bucket_rows(h, w, owners, rows, dir, with_mag, lib)
    if with_mag:
        return tuple(v.reshape(N, m, n) for v in res)
    return res.reshape(N, m, n)


def allreduce(h, w, lib=None):
    """AR = sum_r H_r . W_r^T over whole [N*m, n] matrices."""
    lib = lib or load()
    h, w = _u16(h), _u16(w)
    N, T, k = h.shape
    n = w.shape[1]
    ar = np.empty((T, n), np.float64)
    lib.orc_allreduce(N, T // N, k, n, h, w, ar)
    return ar


def round_bf16(values, lib=None):
    """Round float64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    lib = lib or load()
    v = np.ascontiguousarray(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib.orc_round_bf16(v.reshape(-1), out.reshape(-1), v.size)
    return out
