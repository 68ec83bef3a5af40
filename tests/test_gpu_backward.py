"""GPU parity of the backward pass (through the C ABI) against the CPU oracle,
and of its building blocks (transpose, batched GEMM, AllGather).

Bars: the transpose and the AllGather move bits, so they are bit-exact.  The
gradients are contractions like the forward ops: on small-integer inputs
every partial sum is an integer below 2^24, so fp32 gradients equal the
oracle bit for bit and bf16 gradients equal its nearest-even rounding; on
N(0,1) / N(0, 0.02^2) inputs |gpu - oracle| <= 1e-5 * sum |a*b| over the
contraction (+ 2^-8 |oracle| for bf16 outputs).  The bulk-overlapped and
the serial schedule, and a caller-provided transposed weight, give bitwise
the same gradients (the same kernels on the same data).
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


def as_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(got_t, ref, mag, dtype, dist):
    if dtype == "f32":
        got = as_f64(got_t)
        if dist == "int":
            assert np.array_equal(got, ref), "max |err| %g" % np.abs(got - ref).max()
        else:
            err = np.abs(got - ref)
            assert (err <= 1e-5 * mag).all(), "worst err/bound %g" % (err / np.maximum(1e-5 * mag, 1e-300)).max()
    else:
        bits = gen.torch_bf16_to_bits(got_t)
        if dist == "int":
            assert np.array_equal(bits, oracle.round_bf16(ref))
        else:
            got = gen.bf16_bits_to_f32(bits).astype(np.float64)
            bound = 1e-5 * mag + 2.0 ** -8 * np.abs(ref)
            err = np.abs(got - ref)
            assert (err <= bound).all(), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()


@pytest.mark.parametrize("batch,rows,cols,ld", [(1, 1, 1, 1), (3, 70, 130, 128), (2, 64, 64, 64), (5, 33, 200, 100),
                                                # 16-byte path (cols and ld multiples of 8): ragged tiles, padding,
                                                # a dst tile of padding only
                                                (3, 70, 136, 72), (2, 100, 200, 104), (1, 8, 8, 8), (1, 5, 16, 136)])
def test_transpose(batch, rows, cols, ld):
    say("transpose", batch, rows, cols, ld)
    src = torch.randint(-30000, 30000, (batch, rows, cols), dtype=torch.int16, device="cuda")
    dst = torch.full((batch, cols, ld), 12345, dtype=torch.int16, device="cuda")
    nat.cm_transpose(src, dst, batch, rows, cols, ld)
    torch.cuda.synchronize()
    s, d = src.cpu().numpy(), dst.cpu().numpy()
    assert np.array_equal(d[:, :, :rows], np.transpose(s, (0, 2, 1)))
    assert (d[:, :, rows:] == 0).all()


@pytest.mark.parametrize("batch,M,N,K,out,dist", [(1, 64, 64, 64, "f32", "int"), (3, 300, 200, 192, "f32", "int"),
                                                  (2, 130, 520, 256, "bf16", "int"), (4, 257, 129, 128, "f32", "normal"),
                                                  (130, 32, 64, 64, "f32", "int")])
def test_batched_gemm(batch, M, N, K, out, dist):
    say("gemm", batch, M, N, K, out, dist)
    rng = np.random.default_rng(batch + M)
    if dist == "int":
        a = gen.f32_to_bf16_bits(rng.integers(-3, 4, (batch, M, K)).astype(np.float32))
        b = gen.f32_to_bf16_bits(rng.integers(-3, 4, (batch, N, K)).astype(np.float32))
    else:
        a = gen.f32_to_bf16_bits(rng.standard_normal((batch, M, K)).astype(np.float32))
        b = gen.f32_to_bf16_bits((rng.standard_normal((batch, N, K)) * 0.02).astype(np.float32))
    at, bt = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(b, "cuda")
    ldc = (N + 7) // 8 * 8  # rows padded so every batch's C starts 16-byte aligned
    cp = torch.full((batch, M, ldc), float("nan"), dtype=torch.float32 if out == "f32" else torch.bfloat16, device="cuda")
    nat.cm_gemm(batch, M, N, K, at, K, M * K, bt, K, N * K, cp, ldc, M * ldc, out)
    torch.cuda.synchronize()
    assert torch.isnan(cp[:, :, N:].float()).all()  # nothing written past N
    c = cp[:, :, :N]
    av, bv = gen.bf16_bits_to_f32(a).astype(np.float64), gen.bf16_bits_to_f32(b).astype(np.float64)
    ref = np.einsum("bik,bjk->bij", av, bv)
    mag = np.einsum("bik,bjk->bij", np.abs(av), np.abs(bv))
    check(c, ref, mag, out, dist)


@pytest.mark.parametrize("N,m,k,n_comm,exec_mode", [(1, 5, 8, 1, "graph"), (4, 33, 72, 1, "graph"),
                                                    (8, 16, 256, 2, "eager"), (3, 7, 64, 3, "graph")])
def test_allgather(N, m, k, n_comm, exec_mode):
    say("allgather", N, m, k, n_comm, exec_mode)
    plan = nat.cm_ring_plan(op="allgather", n_ranks=N, m=m, k=k, n=0, n_comm=n_comm, exec_mode=exec_mode)
    x = torch.randint(-30000, 30000, (N, m, k), dtype=torch.int16, device="cuda")
    y = torch.zeros((N, N * m, k), dtype=torch.int16, device="cuda")
    nat.cm_allgather(plan, x, y, torch.cuda.current_stream(), buffers.comm_streams(n_comm))
    torch.cuda.synchronize()
    xs = x.cpu().numpy().reshape(N * m, k)
    for r in range(N):
        assert np.array_equal(y[r].cpu().numpy(), xs)


def run_backward(kind, N, m, k, n, dist, dtype="f32", dir="uni", chunks=1, bulk=True, exec_mode="graph",
                 seed=0, with_wt=False, tensors=None):
    plan = nat.cm_plan_backward(kind=kind, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, n_comm=1, bulk=bulk,
                                dx_dtype=dtype, dw_dtype=dtype, exec_mode=exec_mode)
    if tensors is None:
        arrs = gen.backward_inputs(kind, N, m, k, n, dist, seed)
        tensors = arrs, [gen.to_torch_bf16(a, "cuda") for a in arrs]
    arrs, (act, w, grad) = tensors
    T = N * m
    odt = torch.float32 if dtype == "f32" else torch.bfloat16
    dact = torch.full((N, m, k) if kind == "col" else (N, T, k), float("nan"), dtype=odt, device="cuda")
    dw = torch.full((N, n, k), float("nan"), dtype=odt, device="cuda")
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    wt = w.transpose(1, 2).contiguous() if with_wt else None
    comm = buffers.comm_streams(3)
    say("  backward %s N=%d m=%d k=%d n=%d %s %s dir=%s c=%d bulk=%d %s wt=%d" % (
        kind, N, m, k, n, dist, dtype, dir, chunks, bulk, exec_mode, with_wt))
    nat.cm_linear_backward(plan, act, w, wt, grad, dact, dw, ws, torch.cuda.current_stream(), comm)
    torch.cuda.synchronize()
    return tensors, dact, dw


BWD = [("col", 2, 64, 128, 64, "uni", 1), ("col", 4, 33, 256, 320, "bi", 2), ("col", 3, 40, 64, 128, "direct", 1),
       ("row", 2, 64, 128, 64, "uni", 1), ("row", 4, 33, 192, 320, "bi", 1), ("row", 3, 40, 64, 128, "direct", 2),
       ("col", 1, 50, 64, 64, "uni", 1), ("row", 1, 50, 64, 64, "uni", 1)]


@pytest.mark.parametrize("kind,N,m,k,n,dir,chunks", BWD)
def test_backward_parity(kind, N, m, k, n, dir, chunks):
    say("backward", kind, N, m, k, n, dir, chunks)
    for dist in ("int", "normal"):
        for dtype in ("f32", "bf16"):
            tensors, dact, dw = run_backward(kind, N, m, k, n, dist, dtype, dir, chunks)
            arrs = tensors[0]
            fn = oracle.col_backward if kind == "col" else oracle.row_backward
            rda, rdw, mda, mdw = fn(*arrs, with_mag=True)
            check(dact, rda, mda, dtype, dist)
            check(dw, rdw, mdw, dtype, dist)


@pytest.mark.parametrize("kind", ["col", "row"])
def test_backward_schedules_agree(kind):
    """Bulk overlap, the serial order, eager execution and a caller-provided
    W^T give bitwise the same gradients."""
    N, m, k, n = 4, 48, 192, 128
    tensors, a0, w0 = run_backward(kind, N, m, k, n, "normal", seed=3)
    for kw in (dict(bulk=False), dict(exec_mode="eager"), dict(with_wt=True), dict(bulk=False, exec_mode="eager")):
        _, a1, w1 = run_backward(kind, N, m, k, n, "normal", seed=3, tensors=tensors, **kw)
        assert torch.equal(a0, a1) and torch.equal(w0, w1), kw


@pytest.mark.parametrize("kind", ["col", "row"])
def test_backward_full_size_sampled(kind):
    """The GPT-3 MLP's two linears (8 ranks, 2048 tokens; fc1: k = 12288,
    n = 6144; fc2: k = 6144, n = 12288), bulk overlap, bf16 gradients:
    sampled rows of both gradients against the oracle."""
    N, m = 8, 256
    k, n = (12288, 6144) if kind == "col" else (6144, 12288)
    ts = gen.backward_inputs_torch(kind, N, m, k, n, "normal", 0, "cuda")
    arrs = [gen.torch_bf16_to_bits(t) for t in ts]
    _, dact, dw = run_backward(kind, N, m, k, n, "normal", "bf16", tensors=(arrs, ts))
    rng = np.random.default_rng(5)
    wr, wf = rng.integers(0, N, 6), rng.integers(0, n, 6)
    if kind == "col":
        qo, qr = rng.integers(0, N, 6), rng.integers(0, m, 6)
        rda, mda, rdw, mdw = oracle.col_backward_rows(*arrs, qo, qr, wr, wf)
        ga = dact[torch.as_tensor(qo), torch.as_tensor(qr)]
    else:
        hr, ht = rng.integers(0, N, 6), rng.integers(0, N * m, 6)
        rda, mda, rdw, mdw = oracle.row_backward_rows(*arrs, hr, ht, wr, wf)
        ga = dact[torch.as_tensor(hr), torch.as_tensor(ht)]
    check(ga, rda, mda, "bf16", "normal")
    check(dw[torch.as_tensor(wr), torch.as_tensor(wf)], rdw, mdw, "bf16", "normal")
