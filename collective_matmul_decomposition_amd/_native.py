"""ctypes binding of libcollmm (include/collmm.h): argument marshalling only.

Every call goes straight to the C ABI; all arithmetic runs in the library's
HIP kernels and copy engines.  There is no fallback: if libcollmm.so is
missing the import of these entry points fails loudly.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcollmm.so")

# enums (collmm.h)
CM_OK, CM_ERR_INVALID_ARG, CM_ERR_SHAPE, CM_ERR_ALIGN, CM_ERR_WORKSPACE, CM_ERR_UNSUPPORTED, CM_ERR_HIP, \
    CM_ERR_CAPACITY = range(8)
CM_OP_AG_GEMM, CM_OP_GEMM_RS, CM_OP_GEMM_RS_PIPE, CM_OP_ALLGATHER = range(4)
CM_BWD_COL, CM_BWD_ROW = range(2)
CM_RING_UNI, CM_RING_BI, CM_RING_DIRECT = range(3)
CM_SCHED_DECOMPOSED, CM_SCHED_NAIVE, CM_SCHED_AUTO = range(3)
CM_BF16, CM_F32 = range(2)
CM_BUF_X, CM_BUF_W, CM_BUF_Y, CM_BUF_WS = range(4)
CM_OPK_GEMM, CM_OPK_COPY, CM_OPK_RECORD, CM_OPK_WAIT, CM_OPK_REDUCE = range(5)
CM_EXEC_GRAPH, CM_EXEC_EAGER = range(2)
CM_COPY_SDMA, CM_COPY_CU, CM_COPY_AUTO = range(3)
CM_ACT_NONE, CM_ACT_GELU = range(2)
CM_SKIP_NONE, CM_SKIP_HOPS, CM_SKIP_GEMMS = range(3)
CM_MAX_RANKS, CM_MAX_CHUNKS, CM_MAX_COMM = 64, 16, 32

EXPORTS = ["cm_ring_plan", "cm_pick_overlap", "cm_workspace_size", "cm_plan_program", "cm_trace_create", "cm_trace_destroy",
           "cm_trace_read", "cm_ag_gemm", "cm_gemm_rs", "cm_attention", "cm_layernorm", "cm_plan_layer",
           "cm_layer_forward", "cm_allgather", "cm_transpose", "cm_gemm", "cm_plan_backward", "cm_linear_backward",
           "cm_gemm_rs_noalloc", "cm_status_string", "cm_last_error", "cm_version"]
CM_NOALLOC_WS_BYTES = 256 << 20


class cm_plan_desc(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int), ("n_ranks", ctypes.c_int), ("m", ctypes.c_int), ("k", ctypes.c_int),
                ("n", ctypes.c_int), ("dir", ctypes.c_int), ("chunks", ctypes.c_int), ("sched", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("n_comm", ctypes.c_int),
                ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("exec_mode", ctypes.c_int),
                ("copy_engine", ctypes.c_int), ("bucket_bf16", ctypes.c_int), ("hop_add", ctypes.c_int),
                ("copy_gbps", ctypes.c_double),
                ("mfma_tflops", ctypes.c_double), ("launch_us", ctypes.c_double), ("act", ctypes.c_int),
                ("share", ctypes.c_int), ("split_k", ctypes.c_int), ("skip", ctypes.c_int),
                ("stress", ctypes.c_int), ("group", ctypes.c_int)]


class cm_plan(ctypes.Structure):
    _fields_ = [("desc", cm_plan_desc), ("chunks", ctypes.c_int), ("n_steps", ctypes.c_int),
                ("arc_cw", ctypes.c_int), ("arc_ccw", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("declined", ctypes.c_int), ("n_ops", ctypes.c_int),
                ("n_jobs", ctypes.c_int), ("n_events", ctypes.c_int), ("ws_bytes", ctypes.c_size_t),
                ("est_gemm_us", ctypes.c_double), ("est_hop_us", ctypes.c_double),
                ("est_total_us", ctypes.c_double), ("split", ctypes.c_int), ("n_launches", ctypes.c_int),
                ("group_len", ctypes.c_int * 64), ("slots", ctypes.c_int)]


class cm_op_rec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("stream", ctypes.c_int), ("event", ctypes.c_int), ("step", ctypes.c_int),
                ("chunk", ctypes.c_int), ("first_job", ctypes.c_int), ("n_jobs", ctypes.c_int),
                ("rows", ctypes.c_int), ("cols", ctypes.c_int), ("depth", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("src_buf", ctypes.c_int), ("dst_buf", ctypes.c_int),
                ("src_off", ctypes.c_size_t), ("dst_off", ctypes.c_size_t), ("bytes", ctypes.c_size_t),
                ("act", ctypes.c_int), ("b_share", ctypes.c_int)]


class cm_job_rec(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int), ("dir", ctypes.c_int), ("index", ctypes.c_int), ("a_buf", ctypes.c_int),
                ("b_buf", ctypes.c_int), ("c_buf", ctypes.c_int), ("in0_buf", ctypes.c_int),
                ("in1_buf", ctypes.c_int), ("a_off", ctypes.c_size_t), ("b_off", ctypes.c_size_t),
                ("c_off", ctypes.c_size_t), ("in0_off", ctypes.c_size_t), ("in1_off", ctypes.c_size_t),
                ("lda", ctypes.c_int), ("ldb", ctypes.c_int), ("ldc", ctypes.c_int), ("ld_in", ctypes.c_int),
                ("c_dtype", ctypes.c_int), ("add_dtype", ctypes.c_int)]


class cm_span(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("stream", ctypes.c_int), ("step", ctypes.c_int), ("chunk", ctypes.c_int),
                ("start_us", ctypes.c_double), ("end_us", ctypes.c_double)]


class cm_layer_desc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in ("n_ranks", "m", "d", "heads", "head_dim", "ffn", "dir", "n_comm",
                                            "copy_engine", "exec_mode", "ag_chunks", "rs_chunks", "proj_chunks",
                                            "out_dtype")] + [("ln_eps", ctypes.c_float)]


class cm_layer_plan(ctypes.Structure):
    _fields_ = [("desc", cm_layer_desc), ("qkv", cm_plan), ("proj", cm_plan), ("fc1", cm_plan), ("fc2", cm_plan)] + \
        [(f, ctypes.c_size_t) for f in ("off_qkv", "off_attn", "off_proj", "off_ln", "off_fc1", "off_ops", "ws_bytes")]


class cm_bwd_desc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in ("kind", "n_ranks", "m", "k", "n", "dir", "chunks", "n_comm", "bulk",
                                            "dx_dtype", "dw_dtype", "exec_mode", "copy_engine")]


class cm_bwd_plan(ctypes.Structure):
    _fields_ = [("desc", cm_bwd_desc), ("dgrad", cm_plan), ("gather", cm_plan)] + \
        [(f, ctypes.c_size_t) for f in ("off_wt", "off_g", "off_gt", "off_ot", "off_ops", "ws_bytes")]


class CMError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _status_name(status), detail))


_lib = None


def lib():
    """The loaded libcollmm (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcollmm.so not found at %s; build it with "
                               "`python -m collective_matmul_decomposition_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cs = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.cm_ring_plan.argtypes = [ctypes.POINTER(cm_plan_desc), ctypes.POINTER(cm_plan)]
        L.cm_workspace_size.argtypes = [ctypes.POINTER(cm_plan), ctypes.POINTER(cs)]
        L.cm_pick_overlap.argtypes = [ctypes.POINTER(cm_plan_desc), ctypes.POINTER(cm_plan_desc), ctypes.POINTER(ci),
                                      ctypes.POINTER(ctypes.c_double)]
        L.cm_plan_program.argtypes = [ctypes.POINTER(cm_plan), ctypes.POINTER(cm_op_rec), ci, ctypes.POINTER(ci),
                                      ctypes.POINTER(cm_job_rec), ci, ctypes.POINTER(ci)]
        L.cm_trace_create.argtypes = [ci, ctypes.POINTER(vp)]
        L.cm_trace_destroy.argtypes = [vp]
        L.cm_trace_read.argtypes = [vp, ctypes.POINTER(cm_span), ci, ctypes.POINTER(ci), ctypes.POINTER(ctypes.c_double)]
        for f in (L.cm_ag_gemm, L.cm_gemm_rs):
            f.argtypes = [ctypes.POINTER(cm_plan), vp, vp, vp, vp, cs, vp, ctypes.POINTER(vp), ci, vp]
        L.cm_gemm_rs_noalloc.argtypes = [ctypes.POINTER(cm_plan), vp, vp, vp, vp, ctypes.POINTER(vp), ci]
        L.cm_attention.argtypes = [vp, vp, ci, ci, ci, ci, ci, vp]
        L.cm_layernorm.argtypes = [vp, vp, ci, ci, ctypes.c_float, vp, vp, vp]
        L.cm_plan_layer.argtypes = [ctypes.POINTER(cm_layer_desc), ctypes.POINTER(cm_layer_plan)]
        L.cm_allgather.argtypes = [ctypes.POINTER(cm_plan), vp, vp, vp, ctypes.POINTER(vp), ci, vp]
        L.cm_transpose.argtypes = [vp, vp, ci, ci, ci, ci, vp]
        ll = ctypes.c_longlong
        L.cm_gemm.argtypes = [ci, ci, ci, ci, vp, ci, ll, vp, ci, ll, vp, ci, ll, ci, vp]
        L.cm_plan_backward.argtypes = [ctypes.POINTER(cm_bwd_desc), ctypes.POINTER(cm_bwd_plan)]
        L.cm_linear_backward.argtypes = [ctypes.POINTER(cm_bwd_plan), vp, vp, vp, vp, vp, vp, vp, cs, vp,
                                         ctypes.POINTER(vp), ci]
        L.cm_layer_forward.argtypes = [ctypes.POINTER(cm_layer_plan), vp, vp, vp, vp, vp, vp, vp, cs, vp,
                                       ctypes.POINTER(vp), ci]
        for name in EXPORTS:
            if name in ("cm_status_string", "cm_last_error", "cm_version"):
                continue
            getattr(L, name).restype = ci
        L.cm_status_string.argtypes = [ci]
        L.cm_status_string.restype = ctypes.c_char_p
        L.cm_last_error.argtypes = []
        L.cm_last_error.restype = ctypes.c_char_p
        L.cm_version.argtypes = []
        L.cm_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _status_name(st):
    try:
        return lib().cm_status_string(st).decode()
    except Exception:  # noqa: BLE001 - naming only
        return str(st)


def _check(st, where):
    if st != CM_OK:
        raise CMError(st, where, lib().cm_last_error().decode())


def last_error():
    return lib().cm_last_error().decode()


def version():
    return lib().cm_version().decode()


_ENUMS = {
    "op": {"ag": CM_OP_AG_GEMM, "rs": CM_OP_GEMM_RS, "rs_pipe": CM_OP_GEMM_RS_PIPE, "allgather": CM_OP_ALLGATHER},
    "bwd": {"col": CM_BWD_COL, "row": CM_BWD_ROW},
    "dir": {"uni": CM_RING_UNI, "bi": CM_RING_BI, "direct": CM_RING_DIRECT},
    "sched": {"decomposed": CM_SCHED_DECOMPOSED, "naive": CM_SCHED_NAIVE, "auto": CM_SCHED_AUTO},
    "dtype": {"bf16": CM_BF16, "f32": CM_F32},
    "exec": {"graph": CM_EXEC_GRAPH, "eager": CM_EXEC_EAGER},
    "copy": {"sdma": CM_COPY_SDMA, "cu": CM_COPY_CU, "auto": CM_COPY_AUTO},
    "hop": {"copy": 0, "add": 1},
    "act": {"none": CM_ACT_NONE, "gelu": CM_ACT_GELU},
    "skip": {"none": CM_SKIP_NONE, "hops": CM_SKIP_HOPS, "gemms": CM_SKIP_GEMMS},
}


def make_desc(op, n_ranks, m, k, n, dir="uni", chunks=0, sched="decomposed", out_dtype="bf16", n_comm=1,
              tile=(0, 0), exec_mode="graph", copy_engine="sdma", bucket="f32", hop="copy", copy_gbps=0.0,
              mfma_tflops=0.0, launch_us=0.0, act="none", share=0, split_k=0, skip="none", stress=0, group=0):
    """A cm_plan_desc from keyword arguments (strings or enum values).  group: steps
    per GEMM launch (0 = cost model, 1 = one step per launch, g = at most g).  share=1:
    one rank's share (virtual rank 0's steps at real shape, split-K GEMMs).
    skip="hops" / "gemms": a timing-only mode that runs the program with its hops
    (or its compute-stream launches) replaced by empty operations."""
    def e(kind, v):
        return _ENUMS[kind][v] if isinstance(v, str) else int(v)
    return cm_plan_desc(op=e("op", op), n_ranks=n_ranks, m=m, k=k, n=n, dir=e("dir", dir), chunks=chunks,
                        sched=e("sched", sched), in_dtype=CM_BF16, out_dtype=e("dtype", out_dtype),
                        n_comm=n_comm, tile_m=tile[0], tile_n=tile[1], exec_mode=e("exec", exec_mode),
                        copy_engine=e("copy", copy_engine), bucket_bf16=1 if bucket == "bf16" else 0,
                        hop_add=e("hop", hop), copy_gbps=copy_gbps,
                        mfma_tflops=mfma_tflops, launch_us=launch_us, act=e("act", act), share=int(share),
                        split_k=int(split_k), skip=e("skip", skip), stress=int(stress), group=int(group))


def cm_ring_plan(desc=None, **kw):
    """cm_ring_plan(desc) or cm_ring_plan(op=..., n_ranks=..., ...) -> cm_plan."""
    if desc is None:
        desc = make_desc(**kw)
    p = cm_plan()
    _check(lib().cm_ring_plan(ctypes.byref(desc), ctypes.byref(p)), "cm_ring_plan")
    return p


def cm_pick_overlap(ag, rs):
    """Which of two candidate collectives to decompose: (choice, (saving_ag_us, saving_rs_us)),
    choice 0 = the AllGather, 1 = the ReduceScatter, -1 = neither.  ag / rs are
    cm_plan_desc values or keyword dicts for make_desc."""
    ag = ag if isinstance(ag, cm_plan_desc) else make_desc(**ag)
    rs = rs if isinstance(rs, cm_plan_desc) else make_desc(**rs)
    choice = ctypes.c_int()
    save = (ctypes.c_double * 2)()
    _check(lib().cm_pick_overlap(ctypes.byref(ag), ctypes.byref(rs), ctypes.byref(choice), save), "cm_pick_overlap")
    return choice.value, (save[0], save[1])


def cm_ring_plan_status(desc):
    """Status code of cm_ring_plan without raising (for error-path tests)."""
    p = cm_plan()
    return lib().cm_ring_plan(ctypes.byref(desc), ctypes.byref(p)), p


def cm_workspace_size(plan):
    n = ctypes.c_size_t()
    _check(lib().cm_workspace_size(ctypes.byref(plan), ctypes.byref(n)), "cm_workspace_size")
    return n.value


def cm_plan_program(plan):
    """(ops, jobs): the plan's program as lists of cm_op_rec / cm_job_rec."""
    n_ops, n_jobs = ctypes.c_int(), ctypes.c_int()
    _check(lib().cm_plan_program(ctypes.byref(plan), None, 0, ctypes.byref(n_ops), None, 0, ctypes.byref(n_jobs)),
           "cm_plan_program")
    ops = (cm_op_rec * max(1, n_ops.value))()
    jobs = (cm_job_rec * max(1, n_jobs.value))()
    _check(lib().cm_plan_program(ctypes.byref(plan), ops, n_ops.value, ctypes.byref(n_ops), jobs, n_jobs.value,
                                 ctypes.byref(n_jobs)), "cm_plan_program")
    return list(ops)[:n_ops.value], list(jobs)[:n_jobs.value]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_BF16, _F32 = "bfloat16", "float32"
_BITS_OF = {_BF16: (_BF16, "int16", "uint16"), _F32: (_F32, "int32", "uint32")}


def _dtype_name(dt):
    return _BF16 if dt == CM_BF16 else _F32


def _expect(t, name, elems, dtype):
    """Host-side check of one tensor argument before a launch: on the GPU,
    contiguous, of element type `dtype` ("bfloat16" / "float32"), and holding at
    least `elems` elements (so the kernels stay inside it).  Raw integer device
    pointers are passed through unchecked."""
    if t is None or isinstance(t, int):
        return
    if getattr(t, "device", None) is None or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    # the element type, or an integer type of the same width holding its bit patterns
    if str(t.dtype).split(".")[-1] not in _BITS_OF[dtype]:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.numel() < elems:
        raise ValueError("%s holds %d elements, the plan needs %d" % (name, t.numel(), elems))


def _expect_bytes(t, name, nbytes):
    if t is None or isinstance(t, int):
        return
    if getattr(t, "device", None) is None or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError("%s must be a contiguous GPU tensor" % name)
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, the plan needs %d" % (name, t.numel() * t.element_size(), nbytes))


def _check_plan_tensors(plan, x, w, y, ws):
    """The layouts of include/collmm.h for cm_ag_gemm / cm_gemm_rs."""
    d = plan.desc
    N, m, k, n = d.n_ranks, d.m, d.k, d.n
    T = N * m
    R = 1 if d.share else N
    if d.op == CM_OP_AG_GEMM:
        xe, ye = N * m * k, R * T * n
    else:
        xe, ye = R * T * k, R * m * n
    _expect(x, "x", xe, _BF16)
    _expect(w, "w", R * n * k, _BF16)
    _expect(y, "y", ye, _dtype_name(d.out_dtype))
    if ws is not None:
        _expect_bytes(ws, "ws", plan.ws_bytes)


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream  # torch.cuda.Stream


class Trace:
    """Owns a cm_trace; pass to cm_ag_gemm / cm_gemm_rs, read after a sync."""

    def __init__(self, capacity=4096):
        h = ctypes.c_void_p()
        _check(lib().cm_trace_create(capacity, ctypes.byref(h)), "cm_trace_create")
        self.handle = h
        self.capacity = capacity

    def read(self):
        n = ctypes.c_int()
        total = ctypes.c_double()
        spans = (cm_span * self.capacity)()
        _check(lib().cm_trace_read(self.handle, spans, self.capacity, ctypes.byref(n), ctypes.byref(total)),
               "cm_trace_read")
        return [(s.kind, s.stream, s.step, s.chunk, s.start_us, s.end_us) for s in spans[:n.value]], total.value

    def close(self):
        if self.handle:
            lib().cm_trace_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def _call(fn, name, plan, x, w, y, ws, ws_bytes, compute, comm, trace):
    _check_plan_tensors(plan, x, w, y, ws)
    comm = list(comm or [])
    arr = (ctypes.c_void_p * max(1, len(comm)))(*[_stream(s) for s in comm])
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = fn(ctypes.byref(plan), _ptr(x), _ptr(w), _ptr(y), _ptr(ws), ws_bytes, _stream(compute), arr, len(comm),
            trace.handle if trace is not None else None)
    _check(st, name)


def cm_ag_gemm(plan, x, w, y, ws, compute, comm, trace=None, ws_bytes=None):
    """AllGather -> GEMM through the C ABI (tensors or raw device pointers)."""
    _call(lib().cm_ag_gemm, "cm_ag_gemm", plan, x, w, y, ws, ws_bytes, compute, comm, trace)


def cm_gemm_rs(plan, x, w, y, ws, compute, comm, trace=None, ws_bytes=None):
    """GEMM -> ReduceScatter through the C ABI (tensors or raw device pointers)."""
    _call(lib().cm_gemm_rs, "cm_gemm_rs", plan, x, w, y, ws, ws_bytes, compute, comm, trace)


def cm_gemm_rs_noalloc(plan, x, w, y, compute, comm):
    """GEMM -> ReduceScatter with the library's static workspace (no allocation)."""
    _check_plan_tensors(plan, x, w, y, None)
    comm = list(comm or [])
    arr = (ctypes.c_void_p * max(1, len(comm)))(*[_stream(s) for s in comm])
    _check(lib().cm_gemm_rs_noalloc(ctypes.byref(plan), _ptr(x), _ptr(w), _ptr(y), _stream(compute), arr, len(comm)),
           "cm_gemm_rs_noalloc")


def cm_gemm_rs_noalloc_status(plan, x=None, w=None, y=None, compute=None, comm=None):
    """Status code of cm_gemm_rs_noalloc without raising (for error-path tests)."""
    comm = list(comm or [])
    arr = (ctypes.c_void_p * max(1, len(comm)))(*[_stream(s) for s in comm])
    return lib().cm_gemm_rs_noalloc(ctypes.byref(plan), _ptr(x), _ptr(w), _ptr(y), _stream(compute), arr, len(comm))


# ------------------------------------------------------------ the layer
def cm_attention(qkv, o, n_ranks, T, heads, head_dim=128, causal=True, stream=None):
    """Attention of every head of every virtual rank (tensors or device pointers)."""
    _check(lib().cm_attention(_ptr(qkv), _ptr(o), n_ranks, T, heads, head_dim, 1 if causal else 0, _stream(stream)),
           "cm_attention")


def cm_attention_status(qkv, o, n_ranks, T, heads, head_dim=128, causal=1, stream=None):
    """Status code of cm_attention without raising (for error-path tests)."""
    return lib().cm_attention(_ptr(qkv), _ptr(o), n_ranks, T, heads, head_dim, causal, _stream(stream))


def cm_layernorm(x, y, rows, cols, eps=1e-5, gamma=None, beta=None, stream=None):
    """LayerNorm of fp32 rows into bf16."""
    _check(lib().cm_layernorm(_ptr(x), _ptr(y), rows, cols, eps, _ptr(gamma), _ptr(beta), _stream(stream)),
           "cm_layernorm")


def cm_layernorm_status(x, y, rows, cols, eps=1e-5, gamma=None, beta=None, stream=None):
    return lib().cm_layernorm(_ptr(x), _ptr(y), rows, cols, eps, _ptr(gamma), _ptr(beta), _stream(stream))


def make_layer_desc(n_ranks, m, d, heads, ffn, head_dim=128, dir="uni", n_comm=1, copy_engine="sdma",
                    exec_mode="graph", ag_chunks=0, rs_chunks=0, proj_chunks=0, out_dtype="f32", ln_eps=0.0):
    def e(kind, v):
        return _ENUMS[kind][v] if isinstance(v, str) else int(v)
    return cm_layer_desc(n_ranks=n_ranks, m=m, d=d, heads=heads, head_dim=head_dim, ffn=ffn, dir=e("dir", dir),
                         n_comm=n_comm, copy_engine=e("copy", copy_engine), exec_mode=e("exec", exec_mode),
                         ag_chunks=ag_chunks, rs_chunks=rs_chunks, proj_chunks=proj_chunks,
                         out_dtype=e("dtype", out_dtype), ln_eps=ln_eps)


def cm_plan_layer(desc=None, **kw):
    """cm_plan_layer(desc) or cm_plan_layer(n_ranks=..., ...) -> cm_layer_plan."""
    if desc is None:
        desc = make_layer_desc(**kw)
    p = cm_layer_plan()
    _check(lib().cm_plan_layer(ctypes.byref(desc), ctypes.byref(p)), "cm_plan_layer")
    return p


def cm_plan_layer_status(desc):
    p = cm_layer_plan()
    return lib().cm_plan_layer(ctypes.byref(desc), ctypes.byref(p)), p


def cm_layer_forward(plan, x, wqkv, wo, w1, w2, out, ws, compute, comm, ws_bytes=None):
    """The layer forward through the C ABI."""
    d = plan.desc
    N, m, dm, H, D, F = d.n_ranks, d.m, d.d, d.heads, d.head_dim, d.ffn
    for t, nm, e in ((x, "x", N * m * dm), (wqkv, "wqkv", N * 3 * H * D * dm), (wo, "wo", N * dm * H * D),
                     (w1, "w1", N * F * dm), (w2, "w2", N * dm * F)):
        _expect(t, nm, e, _BF16)
    _expect(out, "out", N * m * dm, _dtype_name(d.out_dtype))
    _expect_bytes(ws, "ws", plan.ws_bytes)
    comm = list(comm or [])
    arr = (ctypes.c_void_p * max(1, len(comm)))(*[_stream(s) for s in comm])
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().cm_layer_forward(ctypes.byref(plan), _ptr(x), _ptr(wqkv), _ptr(wo), _ptr(w1), _ptr(w2), _ptr(out),
                                  _ptr(ws), ws_bytes, _stream(compute), arr, len(comm)), "cm_layer_forward")


# ------------------------------------------------------------ backward
def cm_allgather(plan, x, y, compute, comm, trace=None):
    """AllGather of the shards x [N, m, k] into y [N, N*m, k] through the C ABI."""
    d = plan.desc
    _expect(x, "x", d.n_ranks * d.m * d.k, _BF16)
    _expect(y, "y", d.n_ranks * d.n_ranks * d.m * d.k, _BF16)
    comm = list(comm or [])
    arr = (ctypes.c_void_p * max(1, len(comm)))(*[_stream(s) for s in comm])
    _check(lib().cm_allgather(ctypes.byref(plan), _ptr(x), _ptr(y), _stream(compute), arr, len(comm),
                              trace.handle if trace is not None else None), "cm_allgather")


def cm_transpose(src, dst, batch, rows, cols, ld_dst=None, stream=None):
    _check(lib().cm_transpose(_ptr(src), _ptr(dst), batch, rows, cols, rows if ld_dst is None else ld_dst,
                              _stream(stream)), "cm_transpose")


def cm_transpose_status(src, dst, batch, rows, cols, ld_dst, stream=None):
    return lib().cm_transpose(_ptr(src), _ptr(dst), batch, rows, cols, ld_dst, _stream(stream))


def cm_gemm(batch, M, N, K, a, lda, stride_a, b, ldb, stride_b, c, ldc, stride_c, out_dtype="f32", stream=None):
    """C_b = A_b . B_b^T for b < batch (bf16 in, fp32 accumulate)."""
    od = _ENUMS["dtype"][out_dtype] if isinstance(out_dtype, str) else int(out_dtype)
    _check(lib().cm_gemm(batch, M, N, K, _ptr(a), lda, stride_a, _ptr(b), ldb, stride_b, _ptr(c), ldc, stride_c, od,
                         _stream(stream)), "cm_gemm")


def cm_gemm_status(batch, M, N, K, a, lda, stride_a, b, ldb, stride_b, c, ldc, stride_c, out_dtype=CM_F32, stream=None):
    return lib().cm_gemm(batch, M, N, K, _ptr(a), lda, stride_a, _ptr(b), ldb, stride_b, _ptr(c), ldc, stride_c,
                         out_dtype, _stream(stream))


def make_bwd_desc(kind, n_ranks, m, k, n, dir="uni", chunks=0, n_comm=1, bulk=True, dx_dtype="f32", dw_dtype="f32",
                  exec_mode="graph", copy_engine="sdma"):
    def e(cat, v):
        return _ENUMS[cat][v] if isinstance(v, str) else int(v)
    return cm_bwd_desc(kind=e("bwd", kind), n_ranks=n_ranks, m=m, k=k, n=n, dir=e("dir", dir), chunks=chunks,
                       n_comm=n_comm, bulk=1 if bulk else 0, dx_dtype=e("dtype", dx_dtype),
                       dw_dtype=e("dtype", dw_dtype), exec_mode=e("exec", exec_mode),
                       copy_engine=e("copy", copy_engine))


def cm_plan_backward(desc=None, **kw):
    if desc is None:
        desc = make_bwd_desc(**kw)
    p = cm_bwd_plan()
    _check(lib().cm_plan_backward(ctypes.byref(desc), ctypes.byref(p)), "cm_plan_backward")
    return p


def cm_plan_backward_status(desc):
    p = cm_bwd_plan()
    return lib().cm_plan_backward(ctypes.byref(desc), ctypes.byref(p)), p


def cm_linear_backward(plan, act, w, wt, grad, dact, dw, ws, compute, comm, ws_bytes=None):
    """Backward of a collective matmul: comm = the input gradient's n_comm
    streams, then the bulk stream, then the bulk AllGather's copy lane."""
    d = plan.desc
    N, m, k, n = d.n_ranks, d.m, d.k, d.n
    T = N * m
    col = d.kind == CM_BWD_COL
    _expect(act, "act", N * (m if col else T) * k, _BF16)
    _expect(grad, "grad", N * (T if col else m) * n, _BF16)
    _expect(w, "w", N * n * k, _BF16)
    _expect(wt, "wt", N * k * n, _BF16)
    _expect(dact, "dact", N * (m if col else T) * k, _dtype_name(d.dx_dtype))
    _expect(dw, "dw", N * n * k, _dtype_name(d.dw_dtype))
    _expect_bytes(ws, "ws", plan.ws_bytes)
    comm = list(comm or [])
    arr = (ctypes.c_void_p * max(1, len(comm)))(*[_stream(s) for s in comm])
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().cm_linear_backward(ctypes.byref(plan), _ptr(act), _ptr(w), _ptr(wt), _ptr(grad), _ptr(dact),
                                    _ptr(dw), _ptr(ws), ws_bytes, _stream(compute), arr, len(comm)),
           "cm_linear_backward")
