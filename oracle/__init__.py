"""CPU fp64 oracle for AllGather->GEMM and GEMM->ReduceScatter.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library under test never does,
and this package imports nothing from it.

Thin ctypes wrapper over liboracle.so (oracle.c).  Inputs are numpy uint16
arrays of bf16 bit patterns; outputs are float64.  Shapes:
    ag_gemm:  x [N, m, k], w [N, n, k]    -> y   [N, N*m, n]
    gemm_rs:  h [N, N*m, k], w [N, n, k]  -> out [N, m, n]
    allreduce: same inputs as gemm_rs     -> ar  [N*m, n]
the sequence-parallel transformer layer around them (attention,
LayerNorm, GELU and the chained layer, sp_layer_rows), and the backward pass
of both collective matmuls (col_backward, row_backward).
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
    lib.orc_attention_rows.restype = None
    lib.orc_attention_rows.argtypes = [ci, ci, ci, ci, ci, u16p, ci, i32p, i32p, i32p, f64p, f64p_or_null]
    lib.orc_layernorm.restype = None
    lib.orc_layernorm.argtypes = [ci, ci, f64p, ctypes.c_double, f64p_or_null, f64p_or_null, f64p]
    lib.orc_gelu.restype = None
    lib.orc_gelu.argtypes = [f64p, f64p, ctypes.c_size_t]
    for name in ("orc_col_backward", "orc_row_backward"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [ci, ci, ci, ci, u16p, u16p, u16p, f64p, f64p, f64p_or_null, f64p_or_null]
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


# ---------------------------------------------------------------- the layer
def bf16_to_f64(bits):
    """bf16 bit patterns -> float64 (exact: a bf16 value is a binary32 value)."""
    b = np.ascontiguousarray(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_rows(qkv, heads, ranks, head_idx, rows, causal=True, with_mag=False, lib=None):
    """Attention output rows (see oracle.c): qkv [N, T, 3*heads*D] bf16 bits;
    sample s is query row rows[s] of head head_idx[s] of rank ranks[s].
    Returns out [ns, D] (and mag [ns, D])."""
    lib = lib or load()
    qkv = _u16(qkv)
    N, T, c3 = qkv.shape
    assert c3 % (3 * heads) == 0
    D = c3 // (3 * heads)
    ranks = np.ascontiguousarray(ranks, np.int32)
    head_idx = np.ascontiguousarray(head_idx, np.int32)
    rows = np.ascontiguousarray(rows, np.int32)
    assert ranks.shape == head_idx.shape == rows.shape and ranks.ndim == 1
    assert ((0 <= ranks) & (ranks < N)).all() and ((0 <= head_idx) & (head_idx < heads)).all()
    assert ((0 <= rows) & (rows < T)).all()
    out = np.empty((len(rows), D), np.float64)
    mag = np.empty_like(out) if with_mag else None
    lib.orc_attention_rows(N, T, heads, D, 1 if causal else 0, qkv, len(rows), ranks, head_idx, rows, out, _ptr(mag))
    return (out, mag) if with_mag else out


def attention(qkv, heads, causal=True, with_mag=False, lib=None):
    """Every output row: [N, T, heads*D] (head h in columns h*D..)."""
    N, T, c3 = np.asarray(qkv).shape
    D = c3 // (3 * heads)
    rank_g, row_g, head_g = np.meshgrid(np.arange(N), np.arange(T), np.arange(heads), indexing="ij")
    res = attention_rows(qkv, heads, rank_g.ravel(), head_g.ravel(), row_g.ravel(), causal, with_mag, lib)
    shape = (N, T, heads * D)
    if with_mag:
        return tuple(v.reshape(shape) for v in res)
    return res.reshape(shape)


def layernorm(x, eps=1e-5, gamma=None, beta=None, lib=None):
    """LayerNorm over the last axis of float64 x (any leading shape)."""
    lib = lib or load()
    x = np.ascontiguousarray(x, np.float64)
    cols = x.shape[-1]
    rows = x.size // cols
    g = None if gamma is None else np.ascontiguousarray(gamma, np.float64)
    b = None if beta is None else np.ascontiguousarray(beta, np.float64)
    assert g is None or g.shape == (cols,)
    assert b is None or b.shape == (cols,)
    y = np.empty_like(x)
    lib.orc_layernorm(rows, cols, x.reshape(rows, cols), float(eps), _ptr(g), _ptr(b), y.reshape(rows, cols))
    return y


def gelu(x, lib=None):
    """GELU (erf form) of float64 values, elementwise."""
    lib = lib or load()
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty_like(x)
    lib.orc_gelu(x.reshape(-1), y.reshape(-1), x.size)
    return y


def sp_layer_rows(x, wqkv, wo, w1, w2, heads, tokens, eps=1e-5, causal=True, lib=None):
    """The sequence-parallel transformer-layer forward at selected tokens.

    Inputs (bf16 bit patterns, the library's layouts):
        x     [N, m, d]          sequence shards (T = N*m tokens)
        wqkv  [N, 3*heads*D, d]  rank r's query/key/value projection (heads
                                 r*heads .. of the layer), one output per row
        wo    [N, d, heads*D]    rank r's slice of the output projection
        w1    [N, f/N, d]        rank r's fc1 columns
        w2    [N, d, f/N]        rank r's fc2 rows
    Chain (each stage the monolithic definition; values that the layer
    stores as bf16 between stages are rounded to bf16, nearest-even):
        QKV_r  = bf16(concat(x) . wqkv_r^T)                 AllGather -> GEMM
        A_r    = bf16(attention(QKV_r))                     per head
        P      = sum_r A_r . wo_r^T                         GEMM -> ReduceScatter
        L      = bf16(LayerNorm(P))                         on the shard
        F_r    = bf16(gelu(concat(L) . w1_r^T))             AllGather -> GEMM
        Out    = sum_r F_r . w2_r^T                         GEMM -> ReduceScatter
    tokens: global token indices g (owner g // m, row g % m of Out_owner).
    Returns a dict of float64 arrays, one row per token: "out" [ns, d], "mag"
    (sum_r sum_k |F_r| |w2_r| of the last contraction), and the stages
    "qkv" [N, R, 3*heads*D] (rounded values of the rows 0..R-1 the sample
    needs: R = max(tokens) + 1 when causal, else T), "attn" [N, ns, heads*D]
    (unrounded), "proj" [ns, d], "ln" [ns, d]
    (rounded values) and "fc1" [N, ns, f/N] (rounded values)."""
    lib = lib or load()
    x, wqkv, wo, w1, w2 = (_u16(a) for a in (x, wqkv, wo, w1, w2))
    N, m, d = x.shape
    T = N * m
    HD = wqkv.shape[1] // 3
    assert wqkv.shape == (N, 3 * HD, d) and HD % heads == 0
    assert wo.shape == (N, d, HD)
    fN = w1.shape[1]
    assert w1.shape == (N, fN, d) and w2.shape == (N, d, fN)
    tokens = np.ascontiguousarray(tokens, np.int64)
    assert tokens.ndim == 1 and ((0 <= tokens) & (tokens < T)).all()
    ns = len(tokens)
    rows_needed = int(tokens.max()) + 1 if causal else T
    xf = bf16_to_f64(x).reshape(T, d)
    qkv = np.empty((N, rows_needed, 3 * HD), np.uint16)
    for r in range(N):
        qkv[r] = round_bf16(xf[:rows_needed] @ bf16_to_f64(wqkv[r]).T, lib)
    rr = np.repeat(np.arange(N), ns * heads)
    tt = np.tile(np.repeat(tokens, heads), N)
    hh = np.tile(np.arange(heads), N * ns)
    attn = attention_rows(qkv, heads, rr, hh, tt, causal, False, lib).reshape(N, ns, HD)
    attn_b = bf16_to_f64(round_bf16(attn, lib))
    proj = np.zeros((ns, d))
    for r in range(N):
        proj += attn_b[r] @ bf16_to_f64(wo[r]).T
    ln = bf16_to_f64(round_bf16(layernorm(proj, eps, lib=lib), lib))
    fc1 = np.empty((N, ns, fN))
    for r in range(N):
        fc1[r] = bf16_to_f64(round_bf16(gelu(ln @ bf16_to_f64(w1[r]).T, lib), lib))
    out = np.zeros((ns, d))
    mag = np.zeros((ns, d))
    for r in range(N):
        w2r = bf16_to_f64(w2[r])
        out += fc1[r] @ w2r.T
        mag += np.abs(fc1[r]) @ np.abs(w2r).T
    return {"out": out, "mag": mag, "qkv": bf16_to_f64(qkv), "attn": attn, "proj": proj, "ln": ln, "fc1": fc1}


# ---------------------------------------------------------------- backward
def col_backward(x, w, dy, with_mag=False, lib=None):
    """Backward of AllGather -> GEMM (see oracle.c): x [N, m, k], w [N, n, k],
    dy [N, N*m, n] -> dx [N, m, k], dw [N, n, k] (and their mags)."""
    lib = lib or load()
    x, w, dy = _u16(x), _u16(w), _u16(dy)
    N, m, k = x.shape
    n = w.shape[1]
    assert w.shape == (N, n, k) and dy.shape == (N, N * m, n)
    dx = np.empty((N, m, k))
    dw = np.empty((N, n, k))
    mx = np.empty_like(dx) if with_mag else None
    mw = np.empty_like(dw) if with_mag else None
    lib.orc_col_backward(N, m, k, n, x, w, dy, dx, dw, _ptr(mx), _ptr(mw))
    return (dx, dw, mx, mw) if with_mag else (dx, dw)


def row_backward(h, w, dout, with_mag=False, lib=None):
    """Backward of GEMM -> ReduceScatter: h [N, N*m, k], w [N, n, k],
    dout [N, m, n] -> dh [N, N*m, k], dw [N, n, k] (and their mags)."""
    lib = lib or load()
    h, w, dout = _u16(h), _u16(w), _u16(dout)
    N, T, k = h.shape
    n = w.shape[1]
    m = T // N
    assert w.shape == (N, n, k) and dout.shape == (N, m, n)
    dh = np.empty((N, T, k))
    dw = np.empty((N, n, k))
    mh = np.empty_like(dh) if with_mag else None
    mw = np.empty_like(dw) if with_mag else None
    lib.orc_row_backward(N, m, k, n, h, w, dout, dh, dw, _ptr(mh), _ptr(mw))
    return (dh, dw, mh, mw) if with_mag else (dh, dw)


def col_backward_rows(x, w, dy, dx_owners, dx_rows, dw_ranks, dw_rows, lib=None):
    """Sampled column-parallel backward: dX_q rows (owner q, row i) through
    the duality dX = GEMM->ReduceScatter(dY, W^T) (gemm_rs_rows), and dW_r
    rows f = dY_r[:, f]^T . Xfull (numpy float64).  Returns (dx [s, k], dx_mag,
    dw [s', k], dw_mag)."""
    x, w, dy = _u16(x), _u16(w), _u16(dy)
    N, m, k = x.shape
    wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))
    dx, dx_mag = gemm_rs_rows(dy, wt, dx_owners, dx_rows, with_mag=True, lib=lib)
    X = bf16_to_f64(x).reshape(N * m, k)
    dw = np.empty((len(dw_rows), k))
    dw_mag = np.empty_like(dw)
    for s, (r, f) in enumerate(zip(dw_ranks, dw_rows)):
        g = bf16_to_f64(dy[r][:, f])
        dw[s] = g @ X
        dw_mag[s] = np.abs(g) @ np.abs(X)
    return dx, dx_mag, dw, dw_mag


def row_backward_rows(h, w, dout, dh_ranks, dh_rows, dw_ranks, dw_rows, lib=None):
    """Sampled row-parallel backward: dH_r rows t through the duality
    dH = AllGather->GEMM(dOut, W^T) (ag_gemm_rows), and dW_r rows j =
    dOutfull[:, j]^T . H_r (numpy float64).  Returns (dh [s, k], dh_mag,
    dw [s', k], dw_mag)."""
    h, w, dout = _u16(h), _u16(w), _u16(dout)
    N, T, k = h.shape
    n = w.shape[1]
    wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))
    dh, dh_mag = ag_gemm_rows(dout, wt, dh_ranks, dh_rows, with_mag=True, lib=lib)
    G = bf16_to_f64(dout).reshape(T, n)
    dw = np.empty((len(dw_rows), k))
    dw_mag = np.empty_like(dw)
    for s, (r, j) in enumerate(zip(dw_ranks, dw_rows)):
        Hr = bf16_to_f64(h[r])
        dw[s] = G[:, j] @ Hr
        dw_mag[s] = np.abs(G[:, j]) @ np.abs(Hr)
    return dh, dh_mag, dw, dw_mag
