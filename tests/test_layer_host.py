"""Host-side checks of the layer entry points (no GPU): argument validation
happens before any HIP call, the layer plan's workspace layout, and the
AllGather->GEMM program with the GELU epilogue, executed on the CPU, equals
the oracle's GELU of the oracle's AllGather->GEMM."""
import ctypes

import numpy as np
import pytest

import oracle
from collective_matmul_decomposition_amd import _native as nat
from collective_matmul_decomposition_amd import inputs as gen

from ring_sim import Sim, buffer_sizes


def test_attention_validation():
    ok = dict(qkv=16, o=32, n_ranks=2, T=64, heads=2, head_dim=128, causal=1)
    for kw, want in [(dict(head_dim=64), nat.CM_ERR_UNSUPPORTED), (dict(qkv=0), nat.CM_ERR_INVALID_ARG),
                     (dict(o=0), nat.CM_ERR_INVALID_ARG), (dict(qkv=24), nat.CM_ERR_ALIGN),
                     (dict(n_ranks=0), nat.CM_ERR_INVALID_ARG), (dict(T=0), nat.CM_ERR_INVALID_ARG),
                     (dict(heads=0), nat.CM_ERR_INVALID_ARG), (dict(causal=2), nat.CM_ERR_INVALID_ARG)]:
        args = dict(ok, **kw)
        assert nat.cm_attention_status(**args) == want, kw
        assert nat.last_error()


def test_layernorm_validation():
    for kw, want in [(dict(cols=6), nat.CM_ERR_SHAPE), (dict(cols=16388), nat.CM_ERR_SHAPE),
                     (dict(rows=0), nat.CM_ERR_SHAPE), (dict(x=0), nat.CM_ERR_INVALID_ARG),
                     (dict(eps=-1.0), nat.CM_ERR_INVALID_ARG), (dict(eps=float("inf")), nat.CM_ERR_INVALID_ARG),
                     (dict(y=40), nat.CM_ERR_ALIGN), (dict(gamma=8), nat.CM_ERR_ALIGN)]:
        args = dict(dict(x=16, y=32, rows=4, cols=64, eps=1e-5, gamma=None, beta=None), **kw)
        assert nat.cm_layernorm_status(**args) == want, kw


def test_activation_only_for_allgather():
    st, _ = nat.cm_ring_plan_status(nat.make_desc("rs", 4, 64, 256, 256, act="gelu"))
    assert st == nat.CM_ERR_UNSUPPORTED
    d = nat.make_desc("ag", 4, 64, 256, 256)
    d.act = 7
    assert nat.cm_ring_plan_status(d)[0] == nat.CM_ERR_INVALID_ARG
    for sched in ("decomposed", "naive"):
        plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=64, k=256, n=256, sched=sched, act="gelu")
        ops, _ = nat.cm_plan_program(plan)
        gemms = [o for o in ops if o.kind == nat.CM_OPK_GEMM]
        assert gemms and all(o.act == nat.CM_ACT_GELU for o in gemms)
    plan = nat.cm_ring_plan(op="rs", n_ranks=4, m=64, k=256, n=256, chunks=2)
    assert all(o.act == nat.CM_ACT_NONE for o in nat.cm_plan_program(plan)[0])


@pytest.mark.parametrize("dir,sched,chunks", [("uni", "decomposed", 1), ("bi", "decomposed", 2),
                                              ("direct", "decomposed", 1), ("uni", "naive", 1)])
def test_gelu_program_equals_oracle(dir, sched, chunks):
    N, m, k, n = 4, 8, 64, 64
    plan = nat.cm_ring_plan(op="ag", n_ranks=N, m=m, k=k, n=n, dir=dir, sched=sched, chunks=chunks, out_dtype="f32",
                            n_comm=2, act="gelu")
    x, w = gen.ag_inputs(N, m, k, n, "normal", seed=3)
    sim = Sim(plan, buffer_sizes(plan), {nat.CM_BUF_X: x, nat.CM_BUF_W: w}).run()
    got = sim.buf[nat.CM_BUF_Y].view(np.float32).reshape(N, N * m, n).astype(np.float64)
    want = oracle.gelu(oracle.ag_gemm(x, w))
    # fp32 storage of the simulated result: half an fp32 spacing
    assert np.allclose(got, want, rtol=2 ** -23, atol=1e-30)


def layer_desc(**kw):
    base = dict(n_ranks=8, m=512, d=8192, heads=8, ffn=3584, ag_chunks=1, rs_chunks=1)
    base.update(kw)
    return nat.make_layer_desc(**base)


def test_layer_plan_layout():
    p = nat.cm_plan_layer(layer_desc())
    N, m, d, H, D, f = 8, 512, 8192, 8, 128, 3584
    T = N * m
    assert p.desc.proj_chunks == 4 and abs(p.desc.ln_eps - 1e-5) < 1e-12
    assert (p.qkv.desc.op, p.qkv.desc.k, p.qkv.desc.n, p.qkv.desc.act) == (nat.CM_OP_AG_GEMM, d, 3 * H * D, 0)
    assert (p.proj.desc.op, p.proj.desc.k, p.proj.desc.n, p.proj.chunks) == (nat.CM_OP_GEMM_RS_PIPE, H * D, d, 4)
    assert p.proj.desc.out_dtype == nat.CM_F32
    assert (p.fc1.desc.op, p.fc1.desc.k, p.fc1.desc.n, p.fc1.desc.act) == (nat.CM_OP_AG_GEMM, d, f, nat.CM_ACT_GELU)
    assert (p.fc2.desc.op, p.fc2.desc.k, p.fc2.desc.n, p.fc2.desc.hop_add) == (nat.CM_OP_GEMM_RS, f, d, 1)
    regions = [(p.off_qkv, N * T * 3 * H * D * 2), (p.off_attn, N * T * H * D * 2), (p.off_proj, N * m * d * 4),
               (p.off_ln, N * m * d * 2), (p.off_fc1, N * T * f * 2)]
    end = 0
    for off, size in regions:
        assert off >= end and off % 256 == 0
        end = off + size
    assert p.off_ops >= end
    assert p.ws_bytes == p.off_ops + max(p.qkv.ws_bytes, p.proj.ws_bytes, p.fc1.ws_bytes, p.fc2.ws_bytes)


def test_layer_plan_validation():
    for kw, want in [(dict(head_dim=64), nat.CM_ERR_UNSUPPORTED), (dict(d=8190), nat.CM_ERR_SHAPE),
                     (dict(ffn=100), nat.CM_ERR_SHAPE), (dict(n_ranks=0), nat.CM_ERR_INVALID_ARG),
                     (dict(out_dtype=3), nat.CM_ERR_UNSUPPORTED), (dict(ln_eps=-1.0), nat.CM_ERR_INVALID_ARG)]:
        st, _ = nat.cm_plan_layer_status(layer_desc(**kw))
        assert st == want, kw


def test_layer_forward_validation_before_hip():
    lib = nat.lib()
    p = nat.cm_plan_layer(layer_desc(n_ranks=2, m=64, d=256, heads=1, ffn=256, n_comm=1))
    comm = (ctypes.c_void_p * 1)(1000)

    def call(plan=p, ptrs=(16, 32, 48, 64, 80, 96, 112), ws_bytes=None):
        wsb = plan.ws_bytes if ws_bytes is None else ws_bytes
        return lib.cm_layer_forward(ctypes.byref(plan), *ptrs, wsb, 4096, comm, 1)

    assert call(ptrs=(0, 32, 48, 64, 80, 96, 112)) == nat.CM_ERR_INVALID_ARG
    assert call(ptrs=(16, 32, 48, 64, 80, 96, 0)) == nat.CM_ERR_INVALID_ARG
    assert call(ptrs=(16, 33, 48, 64, 80, 96, 112)) == nat.CM_ERR_ALIGN
    assert call(ws_bytes=p.ws_bytes - 1) == nat.CM_ERR_WORKSPACE
    bad = nat.cm_layer_plan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(p), ctypes.sizeof(p))
    bad.fc1.desc.k += 64  # a plan cm_plan_layer did not make
    assert call(plan=bad) == nat.CM_ERR_INVALID_ARG
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(p), ctypes.sizeof(p))
    bad.off_ln += 256
    assert call(plan=bad) == nat.CM_ERR_INVALID_ARG
