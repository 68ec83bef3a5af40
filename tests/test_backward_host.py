"""Host-side checks of the backward entry points (no GPU): the AllGather
program on the CPU equals concatenation and is race-free, the backward plans'
workspace layout, and argument validation before any HIP call."""
import ctypes

import numpy as np
import pytest

from collective_matmul_decomposition_amd import _native as nat
from collective_matmul_decomposition_amd import inputs as gen

from ring_sim import Sim, buffer_sizes, check_program_bounds


@pytest.mark.parametrize("N,m,k,n_comm", [(1, 3, 8, 1), (2, 5, 16, 1), (3, 4, 64, 2), (5, 2, 24, 3), (8, 3, 64, 8)])
def test_allgather_program(N, m, k, n_comm):
    plan = nat.cm_ring_plan(op="allgather", n_ranks=N, m=m, k=k, n=0, n_comm=n_comm)
    assert plan.ws_bytes == 0
    x = gen.f32_to_bf16_bits(np.random.default_rng(N).integers(-9, 10, (N, m, k)).astype(np.float32))
    sim = Sim(plan, buffer_sizes(plan), {nat.CM_BUF_X: x}).run()
    y = sim.buf[nat.CM_BUF_Y].view(np.uint16).reshape(N, N * m, k)
    for r in range(N):
        assert np.array_equal(y[r], x.reshape(N * m, k))
    assert (sim.writes[nat.CM_BUF_Y] == 1).all()
    ops, _ = nat.cm_plan_program(plan)
    assert all(o.kind != nat.CM_OPK_GEMM for o in ops)
    check_program_bounds(plan)


def test_allgather_validation():
    for kw in (dict(n=64), dict(k=12), dict(m=0), dict(dir="bi"), dict(chunks=2), dict(act="gelu"), dict(hop="add")):
        base = dict(op="allgather", n_ranks=4, m=4, k=64, n=0)
        base.update(kw)
        st, _ = nat.cm_ring_plan_status(nat.make_desc(**base))
        assert st != nat.CM_OK, kw


def test_backward_plans():
    for kind in ("col", "row"):
        p = nat.cm_plan_backward(kind=kind, n_ranks=8, m=256, k=12288, n=6144, chunks=1, n_comm=1)
        N, m, k, n, T = 8, 256, 12288, 6144, 2048
        if kind == "col":
            assert (p.dgrad.desc.op, p.dgrad.desc.k, p.dgrad.desc.n, p.dgrad.desc.hop_add) == (nat.CM_OP_GEMM_RS, n, k, 1)
            assert p.gather.desc.k == k
        else:
            assert (p.dgrad.desc.op, p.dgrad.desc.k, p.dgrad.desc.n) == (nat.CM_OP_AG_GEMM, n, k)
            assert p.gather.desc.k == n
        gk, ok = (k, n) if kind == "col" else (n, k)
        regions = [(p.off_wt, N * n * k * 2), (p.off_g, N * T * gk * 2), (p.off_gt, N * gk * T * 2),
                   (p.off_ot, N * ok * T * 2)]
        end = 0
        for off, size in regions:
            assert off >= end and off % 256 == 0
            end = off + size
        assert p.off_ops >= end and p.ws_bytes == p.off_ops + p.dgrad.ws_bytes
        check_program_bounds(p.dgrad)
        check_program_bounds(p.gather)
        # the ring hops use the requested engine; the per-rank copies of the
        # weight gradient's gather always use the copy kernel
        for ce in ("sdma", "cu"):
            q = nat.cm_plan_backward(kind=kind, n_ranks=4, m=64, k=256, n=128, copy_engine=ce)
            assert q.dgrad.desc.copy_engine == nat._ENUMS["copy"][ce]
            assert q.gather.desc.copy_engine == nat.CM_COPY_CU
    # ragged token count: the weight gradient's operands are padded to 64 tokens
    p = nat.cm_plan_backward(kind="col", n_ranks=3, m=7, k=64, n=128)
    assert p.off_ot - p.off_gt >= 3 * 64 * 64 * 2


def test_backward_plan_validation():
    base = dict(kind="col", n_ranks=4, m=8, k=64, n=128)
    for kw, want in [(dict(kind=5), nat.CM_ERR_INVALID_ARG), (dict(bulk=2), nat.CM_ERR_INVALID_ARG),
                     (dict(k=100), nat.CM_ERR_SHAPE), (dict(n=96), nat.CM_ERR_SHAPE),
                     (dict(dx_dtype=7), nat.CM_ERR_UNSUPPORTED), (dict(n_ranks=0), nat.CM_ERR_INVALID_ARG)]:
        d = nat.make_bwd_desc(**dict(base, **{k: v for k, v in kw.items() if k not in ("kind", "bulk", "dx_dtype")}))
        if "kind" in kw:
            d.kind = kw["kind"]
        if "bulk" in kw:
            d.bulk = kw["bulk"]
        if "dx_dtype" in kw:
            d.dx_dtype = kw["dx_dtype"]
        st, _ = nat.cm_plan_backward_status(d)
        assert st == want, kw


def test_backward_call_validation_before_hip():
    lib = nat.lib()
    p = nat.cm_plan_backward(kind="row", n_ranks=2, m=64, k=128, n=64, n_comm=1)

    def call(plan=p, ptrs=(16, 32, 0, 48, 64, 80, 96), n_comm=3, comm=(1000, 1016, 1032), ws_bytes=None):
        arr = (ctypes.c_void_p * len(comm))(*comm)
        wsb = plan.ws_bytes if ws_bytes is None else ws_bytes
        return lib.cm_linear_backward(ctypes.byref(plan), *ptrs, wsb, 4096, arr, n_comm)

    assert call(ptrs=(0, 32, 0, 48, 64, 80, 96)) == nat.CM_ERR_INVALID_ARG
    assert call(ptrs=(16, 32, 8, 48, 64, 80, 96)) == nat.CM_ERR_ALIGN
    assert call(ws_bytes=p.ws_bytes - 1) == nat.CM_ERR_WORKSPACE
    assert call(n_comm=2, comm=(1000, 1016)) == nat.CM_ERR_INVALID_ARG
    assert call(comm=(1000, 1000, 1032)) == nat.CM_ERR_INVALID_ARG
    assert call(comm=(1000, 4096, 1032)) == nat.CM_ERR_INVALID_ARG
    bad = nat.cm_bwd_plan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(p), ctypes.sizeof(p))
    bad.off_gt += 256
    assert call(plan=bad) == nat.CM_ERR_INVALID_ARG


def test_transpose_and_gemm_validation():
    assert nat.cm_transpose_status(16, 32, 0, 4, 4, 4) == nat.CM_ERR_SHAPE
    assert nat.cm_transpose_status(16, 32, 1, 4, 4, 3) == nat.CM_ERR_SHAPE
    assert nat.cm_transpose_status(0, 32, 1, 4, 4, 4) == nat.CM_ERR_INVALID_ARG
    assert nat.cm_transpose_status(17, 32, 1, 4, 4, 4) == nat.CM_ERR_ALIGN
    g = nat.cm_gemm_status
    assert g(1, 64, 64, 100, 16, 128, 0, 32, 128, 0, 48, 64, 0) == nat.CM_ERR_SHAPE      # K not a multiple of 64
    assert g(1, 64, 64, 64, 16, 60, 0, 32, 64, 0, 48, 64, 0) == nat.CM_ERR_SHAPE         # lda < K
    assert g(1, 64, 64, 64, 16, 64, 0, 32, 64, 0, 48, 64, 0, 9) == nat.CM_ERR_UNSUPPORTED
    assert g(1, 64, 64, 64, 0, 64, 0, 32, 64, 0, 48, 64, 0) == nat.CM_ERR_INVALID_ARG
    assert g(1, 64, 64, 64, 24, 64, 0, 32, 64, 0, 48, 64, 0) == nat.CM_ERR_ALIGN
