"""GPU: the headline (GPT-3-175B MLP) configuration on integer inputs, bit for
bit; the measurement modes; calls on a capturing stream are refused.

Integer inputs in {-3..3} make every fp32 partial sum an exact integer below
2^24 (9 * 12288 < 2^24), so the decomposed result must equal the oracle's
monolithic AllGather-then-GEMM and GEMM-then-ReduceScatter exactly, in the
launch configuration the benchmark times (one comm lane, one chunk per op,
SDMA hops, add-and-forward ReduceScatter hops), on one-way and bidirectional
rings ("Why it works" on the decomposition page: the decomposition is exact by
linearity).
"""
import sys

import numpy as np
import pytest

import oracle
from collective_matmul_decomposition_amd import _native as nat
from collective_matmul_decomposition_amd import buffers
from collective_matmul_decomposition_amd import inputs as gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nat.lib()
    yield


N, T, D, F = 8, 2048, 12288, 49152
M, FN = T // N, F // N
ROWS = 64  # sampled output rows per op


def exact_rows(op, x_t, w_t, y, seed):
    a, w = gen.torch_bf16_to_bits(x_t), gen.torch_bf16_to_bits(w_t)
    rng = np.random.default_rng(seed)
    if op == "ag":
        ranks, rows = rng.integers(0, N, ROWS), rng.integers(0, T, ROWS)
        ref = oracle.ag_gemm_rows(a, w, ranks, rows)
    else:
        ranks, rows = rng.integers(0, N, ROWS), rng.integers(0, M, ROWS)
        ref = oracle.gemm_rs_rows(a, w, ranks, rows)
    got = y.cpu().numpy()[(ranks, rows)].astype(np.float64)
    assert np.array_equal(got, ref), "max |err| %g on %d rows" % (np.abs(got - ref).max(), ROWS)


@pytest.mark.parametrize("dir", ["uni", "bi"])
@pytest.mark.parametrize("op", ["ag", "rs"])
def test_headline_integer_bit_exact(op, dir):
    k, n = (D, FN) if op == "ag" else (FN, D)
    hop = "add" if op == "rs" else "copy"
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=M, k=k, n=n, dir=dir, chunks=1, out_dtype="f32", n_comm=1,
                            copy_engine="sdma", hop=hop)
    mk = gen.ag_inputs_torch if op == "ag" else gen.rs_inputs_torch
    x_t, w_t = mk(N, M, k, n, "int", 7, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    y.fill_(float("nan"))
    say("headline int", op, dir, "chunks", plan.chunks, "tile", plan.tile_m, plan.tile_n)
    comm = buffers.comm_streams(1)
    for rep in range(2):  # the second call replays the cached graph
        buffers.run(plan, x_t, w_t, y, ws, comm=comm)
        torch.cuda.synchronize()
        exact_rows(op, x_t, w_t, y, seed=11 + rep)


def test_capturing_stream_is_refused():
    """A call whose compute or comm stream is being captured into a graph
    returns CM_ERR_UNSUPPORTED and enqueues nothing."""
    plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=64, k=256, n=256, out_dtype="f32", n_comm=1)
    a, w = gen.ag_inputs(4, 64, 256, 256, "int", 0)
    x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    s = torch.cuda.Stream()
    comm = buffers.comm_streams(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    statuses = []
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        for compute, lanes in ((s, comm), (comm[0], [s])):
            arr = (nat.ctypes.c_void_p * 1)(lanes[0].cuda_stream)
            statuses.append(nat.lib().cm_ag_gemm(nat.ctypes.byref(plan), x_t.data_ptr(), w_t.data_ptr(),
                                                 y.data_ptr(), ws.data_ptr(), ws.numel(), compute.cuda_stream, arr,
                                                 1, None))
    assert statuses == [nat.CM_ERR_UNSUPPORTED] * 2, statuses
    assert "captured" in nat.last_error()
    torch.cuda.synchronize()
    # outside the capture the same call runs
    buffers.run(plan, x_t, w_t, y, ws, comm=comm)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.ag_gemm(a, w))


@pytest.mark.parametrize("exec_mode", ["graph", "eager"])
@pytest.mark.parametrize("op", ["ag", "rs"])
def test_measurement_modes(op, exec_mode):
    """skip=hops runs only the GEMMs: for the AllGather each rank's own shard
    (step 0 reads the caller's x) is right and the rest of y is what the
    caller left; skip=gemms runs only the hops and leaves y alone."""
    Nn, m, k, n = 4, 64, 256, 256
    if op == "ag":
        a, w = gen.ag_inputs(Nn, m, k, n, "int", 1)
    else:
        a, w = gen.rs_inputs(Nn, m, k, n, "int", 1)
    x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    ref = oracle.ag_gemm(a, w) if op == "ag" else oracle.gemm_rs(a, w)
    for skip in ("hops", "gemms"):
        plan = nat.cm_ring_plan(op=op, n_ranks=Nn, m=m, k=k, n=n, out_dtype="f32", n_comm=1, exec_mode=exec_mode,
                                hop="add" if op == "rs" else "copy", skip=skip)
        y, ws = buffers.alloc_outputs(plan)
        y.fill_(float("nan"))
        ws.zero_()  # the RS owners' final GEMMs add buckets that no hop filled
        say("skip", skip, op, exec_mode)
        buffers.run(plan, x_t, w_t, y, ws)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        grouped_rs = op == "rs" and any(plan.group_len[i] > 1 for i in range(plan.n_launches))
        if skip == "gemms" and grouped_rs:
            assert not np.isnan(got).any()  # the final add (a comm-stream op) wrote Out from the zeroed workspace
        elif skip == "gemms":
            assert np.isnan(got).all()
        elif op == "ag":
            for r in range(Nn):
                assert np.array_equal(got[r, r * m:(r + 1) * m], ref[r, r * m:(r + 1) * m])
        elif grouped_rs:
            assert np.isnan(got).all()  # grouped steps: Out comes from the final add, a comm-stream op
        else:
            assert not np.isnan(got).any()  # the owners' final GEMMs wrote Out


@pytest.mark.parametrize("dir", ["uni", "bi"])
@pytest.mark.parametrize("op", ["ag", "rs"])
def test_headline_grouped_launches(op, dir):
    """Steps grouped per launch at the headline shape, every grouping limit:
    integer inputs bit-exact on sampled rows, and on real-valued inputs the
    same bits as one step per launch (each output element is the same fp32
    sum in the same order: an AllGather output element comes from one job's K
    loop; a ReduceScatter bucket gets the same additions in ring order)."""
    k, n = (D, FN) if op == "ag" else (FN, D)
    hop = "add" if op == "rs" else "copy"
    mk = gen.ag_inputs_torch if op == "ag" else gen.rs_inputs_torch
    xi, wi = mk(N, M, k, n, "int", 3, "cuda")
    xf, wf = mk(N, M, k, n, "normal", 5, "cuda")
    comm = buffers.comm_streams(1)
    base = None
    for g in (1, 2, 3, 4):
        plan = nat.cm_ring_plan(op=op, n_ranks=N, m=M, k=k, n=n, dir=dir, chunks=1, out_dtype="f32", n_comm=1,
                                copy_engine="sdma", hop=hop, group=g)
        say("grouped", op, dir, "group", g, "launches", list(plan.group_len[:plan.n_launches]))
        y, ws = buffers.alloc_outputs(plan)
        y.fill_(float("nan"))
        buffers.run(plan, xi, wi, y, ws, comm=comm)
        torch.cuda.synchronize()
        exact_rows(op, xi, wi, y, seed=20 + g)
        y.fill_(float("nan"))
        buffers.run(plan, xf, wf, y, ws, comm=comm)
        torch.cuda.synchronize()
        if base is None:
            base = y.clone()
        else:
            assert torch.equal(y, base), "group %d differs from one step per launch" % g
