"""GPU parity: libcollmm (through its C ABI) against the CPU oracle.

Bar (the decomposition is exact by linearity, "Why it works" on the
decomposition page):
  * small-integer inputs: fp32 outputs equal the oracle bit for bit (every
    partial sum is an integer below 2^24, exact in fp32 in any order); bf16
    outputs equal the oracle rounded to nearest-even bf16;
  * bf16 N(0,1) / N(0, 0.02^2) inputs: |gpu - oracle| <= 1e-5 * S, where
    S = sum_k |a_ik * b_kj| over the full contraction, plus 2^-8 |oracle| for
    bf16 outputs;
  * repeated runs are bitwise identical (no atomics).
Shapes span several tiles with ragged tails, every schedule (uni / bi ring,
naive, pipeline chunks), several chunk and comm-stream counts, N = 1 and
N = 2 degenerate rings, and the full-size Llama-3-8B and GPT-3 MLP shapes on
sampled rows.
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
    nat.lib()  # fail loudly if the library is missing
    yield


def run_case(op, N, m, k, n, dist="int", out="f32", dir="uni", chunks=1, sched="decomposed", n_comm=1, seed=0,
             repeat=1, tile=(0, 0), exec_mode="graph", copy_engine="sdma", hop="copy"):
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, sched=sched, out_dtype=out,
                            n_comm=n_comm, tile=tile, exec_mode=exec_mode, copy_engine=copy_engine, hop=hop)
    if op == "ag":
        a, w = gen.ag_inputs(N, m, k, n, dist, seed)
    else:
        a, w = gen.rs_inputs(N, m, k, n, dist, seed)
    x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    comm = buffers.comm_streams(n_comm)
    results = []
    for _ in range(repeat):
        say("  launch %s N=%d m=%d k=%d n=%d %s out=%s dir=%s c=%d(%d) sched=%s n_comm=%d tile=%dx%d %s" %
            (op, N, m, k, n, dist, out, dir, chunks, plan.chunks, sched, n_comm, plan.tile_m, plan.tile_n, exec_mode))
        y.fill_(float("nan")) if out == "f32" else y.fill_(float("nan"))
        buffers.run(plan, x_t, w_t, y, ws, comm=comm)
        torch.cuda.synchronize()
        results.append(y.detach().clone())
    return plan, a, w, results


def check(op, a, w, y, out, dist):
    ref, mag = (oracle.ag_gemm if op == "ag" else oracle.gemm_rs)(a, w, with_mag=True)
    if out == "f32":
        got = y.float().cpu().numpy().astype(np.float64)
        if dist == "int":
            assert np.array_equal(got, ref), "max |err| %g" % np.abs(got - ref).max()
        else:
            err = np.abs(got - ref)
            bound = 1e-5 * mag
            assert (err <= bound).all(), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()
    else:
        bits = gen.torch_bf16_to_bits(y)
        if dist == "int":
            assert np.array_equal(bits, oracle.round_bf16(ref))
        else:
            got = gen.bf16_bits_to_f32(bits).astype(np.float64)
            err = np.abs(got - ref)
            bound = 1e-5 * mag + 2.0 ** -8 * np.abs(ref)
            assert (err <= bound).all(), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()


# the tiny configuration: N = 4, 256 tokens (64-row shards), d = 256, ffn 1024 (f/N = 256)
TINY = []
for op in ("ag", "rs", "rs_pipe"):
    for dir, sched, chunks in (("uni", "decomposed", 1), ("uni", "decomposed", 2), ("bi", "decomposed", 1),
                               ("bi", "decomposed", 2), ("uni", "naive", 1)):
        if op == "rs_pipe" and (dir == "bi" or sched == "naive"):
            continue
        for dist in ("int", "normal"):
            for out in ("f32", "bf16"):
                TINY.append((op, dir, sched, chunks, dist, out))


@pytest.mark.parametrize("exec_mode,copy_engine", [("graph", "sdma"), ("eager", "sdma"), ("graph", "cu"),
                                                   ("eager", "cu")])
@pytest.mark.parametrize("op,dir,sched,chunks,dist,out", TINY)
def test_tiny_config(op, dir, sched, chunks, dist, out, exec_mode, copy_engine):
    say("tiny", op, dir, sched, chunks, dist, out, exec_mode, copy_engine)
    _, a, w, (y,) = run_case(op, 4, 64, 256, 256, dist, out, dir, chunks, sched, n_comm=4, exec_mode=exec_mode,
                             copy_engine=copy_engine)
    check(op, a, w, y, out, dist)


RAGGED = [
    # op, N, m, k, n, dir, chunks, n_comm
    ("ag", 3, 40, 192, 320, "uni", 2, 2),
    ("ag", 5, 100, 128, 448, "bi", 1, 3),
    ("ag", 1, 70, 64, 64, "uni", 1, 1),
    ("ag", 2, 33, 320, 960, "bi", 1, 2),
    ("rs", 3, 37, 192, 320, "uni", 5, 2),
    ("rs", 5, 21, 128, 448, "bi", 7, 4),
    ("rs", 1, 50, 64, 128, "uni", 2, 1),
    ("rs", 2, 19, 256, 640, "uni", 2, 2),
    ("rs_pipe", 3, 29, 192, 384, "uni", 3, 3),
    ("rs_pipe", 6, 17, 64, 256, "uni", 4, 6),
    ("rs_pipe", 1, 30, 128, 128, "uni", 2, 1),
]


@pytest.mark.parametrize("op,N,m,k,n,dir,chunks,n_comm", RAGGED)
def test_ragged_shapes(op, N, m, k, n, dir, chunks, n_comm):
    say("ragged", op, N, m, k, n, dir, chunks, n_comm)
    for dist, out in (("int", "f32"), ("normal", "bf16")):
        _, a, w, (y,) = run_case(op, N, m, k, n, dist, out, dir, chunks, "decomposed", n_comm)
        check(op, a, w, y, out, dist)


# The limits: 64 virtual ranks (CM_MAX_RANKS) with one to three rows per shard,
# on every schedule (so launches of 64 and 128 jobs, and the pipeline's 4096
# jobs split over launches), and the maximum of 16 chunks.
EXTREME = [
    # op, N, m, k, n, dir, chunks, n_comm, hop
    ("ag", 64, 1, 64, 64, "uni", 1, 4, "copy"),
    ("ag", 64, 2, 64, 128, "bi", 2, 8, "copy"),
    ("rs", 64, 3, 64, 64, "uni", 1, 4, "copy"),
    ("rs", 64, 1, 64, 64, "bi", 1, 8, "copy"),
    ("rs", 64, 2, 64, 64, "uni", 1, 4, "add"),
    ("rs_pipe", 64, 2, 64, 128, "uni", 2, 4, "copy"),
    ("ag", 64, 1, 64, 64, "direct", 1, 4, "copy"),
    ("rs", 64, 1, 64, 64, "direct", 1, 4, "copy"),
    ("ag", 4, 32, 64, 64, "uni", 16, 2, "copy"),
    ("rs", 3, 8, 64, 1024, "uni", 16, 2, "copy"),
    ("rs", 3, 8, 64, 1024, "bi", 16, 3, "add"),
]


@pytest.mark.parametrize("op,N,m,k,n,dir,chunks,n_comm,hop", EXTREME)
def test_extreme_shapes(op, N, m, k, n, dir, chunks, n_comm, hop):
    say("extreme", op, N, m, k, n, dir, chunks, n_comm, hop)
    for dist, out in (("int", "f32"), ("normal", "bf16")):
        _, a, w, (y,) = run_case(op, N, m, k, n, dist, out, dir, chunks, "decomposed", n_comm, hop=hop)
        check(op, a, w, y, out, dist)


MID = [("ag", "uni", 1), ("ag", "bi", 2), ("rs", "uni", 2), ("rs", "bi", 4), ("rs_pipe", "uni", 4)]


@pytest.mark.parametrize("op,dir,chunks", MID)
def test_mid_size_eight_ranks(op, dir, chunks):
    """N = 8, 2048 tokens, several 256x256 tiles per rank and step."""
    N, m = 8, 256
    k, n = (1024, 768) if op == "ag" else (768, 1024)
    say("mid", op, dir, chunks)
    _, a, w, (y,) = run_case(op, N, m, k, n, "int", "f32", dir, chunks, "decomposed", n_comm=8)
    check(op, a, w, y, "f32", "int")


TILES = [(256, 256), (256, 192), (256, 128), (128, 256), (128, 128), (64, 256)]


@pytest.mark.parametrize("tile", TILES, ids=lambda t: "%dx%d" % t)
@pytest.mark.parametrize("op", ["ag", "rs"])
def test_every_tile_variant(tile, op):
    """Each compiled block tile, forced, on a shape with ragged rows and columns."""
    N, m, k = 3, 300, 192
    n = 320 if op == "ag" else 640
    say("tile", tile, op)
    for dist, out in (("int", "f32"), ("normal", "bf16")):
        _, a, w, (y,) = run_case(op, N, m, k, n, dist, out, "uni", 1 if op == "ag" else 2, "decomposed", 2,
                                 tile=tile)
        check(op, a, w, y, out, dist)


@pytest.mark.parametrize("op", ["ag", "rs", "rs_pipe"])
def test_repeatable_bitwise(op):
    """Graph replays (the second and third call reuse the captured graph) and
    the eager path give bit-identical results."""
    say("repeat", op)
    n = 512 if op != "ag" else 384
    _, _, _, ys = run_case(op, 4, 128, 512, n, "normal", "f32", "uni", 2, "decomposed", 4, repeat=3)
    _, _, _, ye = run_case(op, 4, 128, 512, n, "normal", "f32", "uni", 2, "decomposed", 4, exec_mode="eager")
    for y in ys[1:] + ye:
        assert torch.equal(y, ys[0])


def test_bi_equals_uni_on_integers():
    for op in ("ag", "rs"):
        say("bi==uni", op)
        _, _, _, (yu,) = run_case(op, 7, 64, 256, 256, "int", "f32", "uni", 2, "decomposed", 7)
        _, _, _, (yb,) = run_case(op, 7, 64, 256, 256, "int", "f32", "bi", 2, "decomposed", 14)
        assert torch.equal(yu, yb)


def test_trace_spans():
    """The timing trace records every GEMM launch and hop with ordered times."""
    plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=64, k=256, n=256, n_comm=4)
    a, w = gen.ag_inputs(4, 64, 256, 256, "int", 0)
    x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    tr = nat.Trace(256)
    say("trace")
    buffers.run(plan, x_t, w_t, y, ws, trace=tr)
    torch.cuda.synchronize()
    spans, total = tr.read()
    kinds = [s[0] for s in spans]
    assert kinds.count(nat.CM_OPK_GEMM) == plan.n_launches  # one span per launch (steps grouped or not)
    assert kinds.count(nat.CM_OPK_COPY) >= 3
    assert all(s[5] >= s[4] >= 0 for s in spans) and total > 0
    tr.close()
    check("ag", a, w, y, "bf16", "int")


FULL = [
    # op, N, m, k, n, dir, n_comm, chunks (0 = cost model)
    # Llama-3-8B MLP: N = 8, 4096 tokens, d = 4096, ffn 14336 (f/N = 1792)
    ("ag", 8, 512, 4096, 1792, "uni", 8, 0),
    ("rs", 8, 512, 1792, 4096, "uni", 8, 0),
    ("rs_pipe", 8, 512, 1792, 4096, "uni", 8, 0),
    ("ag", 8, 512, 4096, 1792, "uni", 1, 1),
    ("rs", 8, 512, 1792, 4096, "uni", 1, 1),
    # GPT-3 175B MLP: N = 8, 2048 tokens, d = 12288, ffn 49152 (f/N = 6144)
    ("ag", 8, 256, 12288, 6144, "uni", 8, 0),
    ("ag", 8, 256, 12288, 6144, "bi", 16, 0),
    ("rs", 8, 256, 6144, 12288, "uni", 8, 0),
    ("rs", 8, 256, 6144, 12288, "bi", 16, 0),
    # the benchmark's launch configuration: one comm lane, one chunk per op
    ("ag", 8, 256, 12288, 6144, "uni", 1, 1),
    ("rs", 8, 256, 6144, 12288, "uni", 1, 1),
    ("rs", 8, 256, 6144, 12288, "uni", 1, 2),
]
FULL_CU = [("ag", 8, 256, 12288, 6144, "uni", 1, 1), ("rs", 8, 256, 6144, 12288, "uni", 1, 1),
           ("ag", 8, 512, 4096, 1792, "uni", 1, 1), ("rs", 8, 512, 1792, 4096, "uni", 1, 1)]


def sampled_check(op, N, m, x_t, w_t, y, n_rows, seed=1, exact=False):
    """Sampled output rows against the oracle: bitwise for integer inputs
    with fp32 outputs (exact=True), else within the stated bound."""
    a, w = gen.torch_bf16_to_bits(x_t), gen.torch_bf16_to_bits(w_t)
    rng = np.random.default_rng(seed)
    if op == "ag":
        ranks = rng.integers(0, N, n_rows)
        rows = rng.integers(0, N * m, n_rows)
        ref, mag = oracle.ag_gemm_rows(a, w, ranks, rows, with_mag=True)
        sel = (ranks, rows)
    else:
        owners = rng.integers(0, N, n_rows)
        rows = rng.integers(0, m, n_rows)
        ref, mag = oracle.gemm_rs_rows(a, w, owners, rows, with_mag=True)
        sel = (owners, rows)
    if y.dtype == torch.float32:
        got = y.cpu().numpy()[sel].astype(np.float64)
        if exact:
            assert np.array_equal(got, ref), "max |err| %g" % np.abs(got - ref).max()
            return
        bound = 1e-5 * mag
    else:
        got = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y)[sel]).astype(np.float64)
        if exact:
            assert np.array_equal(gen.torch_bf16_to_bits(y)[sel], oracle.round_bf16(ref))
            return
        bound = 1e-5 * mag + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    assert (err <= bound).all(), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()


@pytest.mark.parametrize("op,N,m,k,n,dir,n_comm,chunks,copy_engine",
                         [f + ("sdma",) for f in FULL] + [f + ("cu",) for f in FULL_CU])
def test_full_size_sampled(op, N, m, k, n, dir, n_comm, chunks, copy_engine):
    """Full-size shapes, including the benchmark's launch configuration; sampled rows against the oracle."""
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype="bf16",
                            n_comm=n_comm, copy_engine=copy_engine)
    mk = gen.ag_inputs_torch if op == "ag" else gen.rs_inputs_torch
    x_t, w_t = mk(N, m, k, n, "normal", 0, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    say("full", op, N, m, k, n, dir, "n_comm", n_comm, "chunks", plan.chunks, "tile", plan.tile_m, plan.tile_n)
    buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(n_comm))
    torch.cuda.synchronize()
    sampled_check(op, N, m, x_t, w_t, y, 12 if op == "ag" else 8)


# The small-chunk regime sweep: d = 2048, ffn 8192, 1024 tokens, N in {2, 4, 8}
# and chunks per shard in {1, 2, 4}, for AG, RS and the pipeline-chunk RS.
C4 = [(op, N, c) for op in ("ag", "rs", "rs_pipe") for N in (2, 4, 8) for c in (1, 2, 4)]


@pytest.mark.parametrize("op,N,c", C4)
def test_small_chunk_sweep(op, N, c):
    T, d, f = 1024, 2048, 8192
    m = T // N
    k, n = (d, f // N) if op == "ag" else (f // N, d)
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, chunks=c, out_dtype="f32", n_comm=1)
    say("c4", op, N, c, "tile", plan.tile_m, plan.tile_n)
    for dist, seed in (("int", 3), ("normal", 4)):
        if op == "ag":
            a, w = gen.ag_inputs(N, m, k, n, dist, seed)
        else:
            a, w = gen.rs_inputs(N, m, k, n, dist, seed)
        x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
        y, ws = buffers.alloc_outputs(plan)
        buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(1))
        torch.cuda.synchronize()
        sampled_check(op, N, m, x_t, w_t, y, 16, seed=seed, exact=(dist == "int"))


# The four GEMM + collective pairs of the SP transformer layer (N = 8, 4096
# tokens, d = 8192, 64 heads, ffn 28672): AG->QKV (f/N = 3072 columns of the
# fused QKV projection), out-proj->pipeline-chunk RS (K = 1024), AG->fc1
# (3584), fc2->RS (K = 3584).
C5 = [("ag", 8192, 3072, 0), ("rs_pipe", 1024, 8192, 4), ("ag", 8192, 3584, 0), ("rs", 3584, 8192, 0)]


@pytest.mark.parametrize("op,k,n,chunks", C5)
def test_layer_gemm_pairs(op, k, n, chunks):
    N, m = 8, 512
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, chunks=chunks, out_dtype="bf16", n_comm=1)
    mk = gen.ag_inputs_torch if op == "ag" else gen.rs_inputs_torch
    x_t, w_t = mk(N, m, k, n, "normal", 5, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    say("c5", op, k, n, "chunks", plan.chunks, "tile", plan.tile_m, plan.tile_n)
    buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(1))
    torch.cuda.synchronize()
    sampled_check(op, N, m, x_t, w_t, y, 12, seed=6)


# GEMM -> ReduceScatter with the bucket held in bf16 between hops.  Integer
# inputs: partial products and bucket sums are exact in fp32, so the GPU
# rounds the same values the oracle rounds and the result is bitwise equal.
# Float inputs: the GPU's fp32 partials differ from the exact ones by at most
# 1e-5 * sum|a*w|, and each bucket rounding can then land on the neighbouring
# bf16 value, at most one spacing (2^-7 of the value) away; the oracle's
# rmag sums |bucket| over every rounding.
BF16B = [
    # N, m, k, n, dir, chunks, out
    (4, 64, 256, 256, "uni", 1, "f32"),
    (4, 64, 256, 256, "bi", 2, "f32"),
    (5, 100, 128, 448, "bi", 1, "bf16"),
    (3, 37, 192, 320, "uni", 5, "f32"),
    (8, 256, 768, 1024, "uni", 2, "f32"),
    (7, 64, 256, 512, "bi", 2, "bf16"),
]


@pytest.mark.parametrize("N,m,k,n,dir,chunks,out", BF16B)
def test_bf16_bucket_rs(N, m, k, n, dir, chunks, out):
    plan = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype=out,
                            n_comm=2, bucket="bf16")
    for dist in ("int", "normal"):
        a, w = gen.rs_inputs(N, m, k, n, dist, 7)
        x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
        y, ws = buffers.alloc_outputs(plan)
        say("bf16 bucket", N, m, k, n, dir, chunks, out, dist)
        buffers.run(plan, x_t, w_t, y, ws)
        torch.cuda.synchronize()
        ref, mag, rmag = oracle.gemm_rs_bf16_bucket(a, w, dir=dir, with_mag=True)
        if out == "f32":
            got = y.cpu().numpy().astype(np.float64)
        else:
            got = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y)).astype(np.float64)
        if dist == "int":
            want = ref if out == "f32" else gen.bf16_bits_to_f32(oracle.round_bf16(ref)).astype(np.float64)
            assert np.array_equal(got, want), "max |err| %g" % np.abs(got - want).max()
        else:
            bound = 1e-5 * mag + 2.0 ** -7 * rmag + (2.0 ** -8 * np.abs(ref) if out == "bf16" else 0)
            err = np.abs(got - ref)
            assert (err <= bound).all(), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()


def test_bf16_bucket_rs_full_size_sampled():
    """The GPT-3 MLP fc2 step with bf16 buckets (one lane, one chunk, as the benchmark runs it)."""
    N, m, k, n = 8, 256, 6144, 12288
    plan = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=k, n=n, chunks=1, out_dtype="bf16", n_comm=1, bucket="bf16")
    x_t, w_t = gen.rs_inputs_torch(N, m, k, n, "normal", 0, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    say("bf16 bucket full")
    buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(1))
    torch.cuda.synchronize()
    a, w = gen.torch_bf16_to_bits(x_t), gen.torch_bf16_to_bits(w_t)
    rng = np.random.default_rng(3)
    owners, rows = rng.integers(0, N, 8), rng.integers(0, m, 8)
    ref, mag, rmag = oracle.gemm_rs_bf16_bucket_rows(a, w, owners, rows, with_mag=True)
    got = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y)[owners, rows]).astype(np.float64)
    bound = 1e-5 * mag + 2.0 ** -7 * rmag + 2.0 ** -8 * np.abs(ref)
    assert (np.abs(got - ref) <= bound).all()


# Direct-peer schedules: owner -> consumer transfers, the ring's order of
# shards and of additions, so the results equal the one-way ring's bitwise.
DIRECT = [
    # op, N, m, k, n, chunks, n_comm
    ("ag", 4, 64, 256, 256, 1, 1),
    ("ag", 5, 100, 128, 448, 2, 3),
    ("ag", 8, 256, 1024, 768, 1, 8),
    ("rs", 4, 64, 256, 256, 1, 1),
    ("rs", 5, 37, 192, 320, 5, 3),
    ("rs", 8, 256, 768, 1024, 2, 8),
    ("rs", 2, 19, 256, 640, 2, 2),
]


@pytest.mark.parametrize("op,N,m,k,n,chunks,n_comm", DIRECT)
def test_direct_schedule_equals_ring(op, N, m, k, n, chunks, n_comm):
    say("direct", op, N, m, k, n, chunks, n_comm)
    _, a, w, (yi,) = run_case(op, N, m, k, n, "int", "f32", "direct", chunks, "decomposed", n_comm)
    check(op, a, w, yi, "f32", "int")
    _, _, _, (yd,) = run_case(op, N, m, k, n, "normal", "f32", "direct", chunks, "decomposed", n_comm, seed=9)
    _, _, _, (yu,) = run_case(op, N, m, k, n, "normal", "f32", "uni", chunks, "decomposed", n_comm, seed=9)
    assert torch.equal(yd, yu)


@pytest.mark.parametrize("op", ["ag", "rs"])
def test_direct_schedule_full_size_sampled(op):
    N, m = 8, 256
    k, n = (12288, 6144) if op == "ag" else (6144, 12288)
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir="direct", chunks=1, out_dtype="bf16", n_comm=1)
    mk = gen.ag_inputs_torch if op == "ag" else gen.rs_inputs_torch
    x_t, w_t = mk(N, m, k, n, "normal", 0, "cuda")
    y, ws = buffers.alloc_outputs(plan)
    say("direct full", op)
    buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(1))
    torch.cuda.synchronize()
    sampled_check(op, N, m, x_t, w_t, y, 8)


@pytest.mark.parametrize("op", ["ag", "rs", "rs_pipe"])
def test_auto_schedule(op):
    """The decline gate's resolved plan (decomposed or naive) runs and matches the oracle."""
    for kw in (dict(), dict(copy_gbps=1.0)):
        plan = nat.cm_ring_plan(op=op, n_ranks=4, m=64, k=256, n=256, sched="auto", out_dtype="f32", n_comm=2, **kw)
        a, w = (gen.ag_inputs if op == "ag" else gen.rs_inputs)(4, 64, 256, 256, "int", 1)
        x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
        y, ws = buffers.alloc_outputs(plan)
        say("auto", op, kw, "resolved", plan.desc.sched, "declined", plan.declined)
        buffers.run(plan, x_t, w_t, y, ws)
        torch.cuda.synchronize()
        check(op, a, w, y, "f32", "int")


HOP_ADD = [
    # N, m, k, n, dir, chunks, n_comm
    (2, 19, 256, 640, "uni", 2, 1),
    (3, 64, 256, 256, "bi", 1, 2),
    (4, 64, 256, 256, "uni", 1, 1),
    (5, 37, 192, 320, "bi", 5, 3),
    (8, 256, 768, 1024, "uni", 2, 1),
    (8, 256, 768, 1024, "bi", 1, 2),
]


@pytest.mark.parametrize("N,m,k,n,dir,chunks,n_comm", HOP_ADD)
def test_hop_add_equals_epilogue_ring(N, m, k, n, dir, chunks, n_comm):
    """Add-and-forward hops: the oracle's bound on integers, and bitwise the
    sums of the ring that adds in the GEMM epilogue on real-valued data."""
    say("hop add", N, m, k, n, dir, chunks, n_comm)
    for out in ("f32", "bf16"):
        _, a, w, (yi,) = run_case("rs", N, m, k, n, "int", out, dir, chunks, "decomposed", n_comm, hop="add")
        check("rs", a, w, yi, out, "int")
    for exec_mode in ("graph", "eager"):
        _, _, _, (ya,) = run_case("rs", N, m, k, n, "normal", "f32", dir, chunks, "decomposed", n_comm, seed=9,
                                  exec_mode=exec_mode, hop="add")
        _, _, _, (yc,) = run_case("rs", N, m, k, n, "normal", "f32", dir, chunks, "decomposed", n_comm, seed=9,
                                  exec_mode=exec_mode)
        assert torch.equal(ya, yc)


PIPE_ADD = [
    # op, N, m, k, n, chunks, n_comm, sched
    ("rs_pipe", 2, 19, 256, 640, 2, 1, "decomposed"),
    ("rs_pipe", 3, 64, 256, 256, 4, 2, "decomposed"),
    ("rs_pipe", 5, 37, 192, 320, 5, 3, "decomposed"),
    ("rs_pipe", 8, 256, 768, 1024, 4, 1, "decomposed"),
    ("rs", 4, 64, 256, 256, 1, 1, "naive"),
    ("rs_pipe", 1, 50, 64, 128, 2, 1, "decomposed"),
]


@pytest.mark.parametrize("op,N,m,k,n,chunks,n_comm,sched", PIPE_ADD)
def test_pipe_hop_add_equals_copy_ring(op, N, m, k, n, chunks, n_comm, sched):
    """Pipeline-chunk (and naive) ReduceScatter with add-and-forward hops:
    exact on integers, and bitwise the sums of the copy-and-add ring."""
    say("pipe hop add", op, N, m, k, n, chunks, n_comm, sched)
    for out in ("f32", "bf16"):
        _, a, w, (yi,) = run_case(op, N, m, k, n, "int", out, "uni", chunks, sched, n_comm, hop="add")
        check("rs", a, w, yi, out, "int")
    for exec_mode in ("graph", "eager"):
        _, a, w, (ya,) = run_case(op, N, m, k, n, "normal", "f32", "uni", chunks, sched, n_comm, seed=9,
                                  exec_mode=exec_mode, hop="add")
        check("rs", a, w, ya, "f32", "normal")
        _, _, _, (yc,) = run_case(op, N, m, k, n, "normal", "f32", "uni", chunks, sched, n_comm, seed=9,
                                  exec_mode=exec_mode)
        assert torch.equal(ya, yc)


def test_pipe_hop_add_layer_shape_sampled():
    """The layer's output projection: 8 ranks, [4096 x 1024] . [1024 x 8192]
    per rank in 4 pipeline chunks, add-and-forward hops, fp32 out: sampled
    rows against the oracle, the whole output bitwise equal to the copy ring's."""
    N, m, k, n = 8, 512, 1024, 8192
    x_t, w_t = gen.rs_inputs_torch(N, m, k, n, "normal", 0, "cuda")
    ys = []
    for hop in ("add", "copy"):
        plan = nat.cm_ring_plan(op="rs_pipe", n_ranks=N, m=m, k=k, n=n, chunks=4, out_dtype="f32", n_comm=1, hop=hop)
        y, ws = buffers.alloc_outputs(plan)
        say("pipe hop full", hop)
        buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(1))
        torch.cuda.synchronize()
        ys.append(y)
        del ws
    sampled_check("rs", N, m, x_t, w_t, ys[0], 8)
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("dir", ["uni", "bi"])
def test_hop_add_full_size_sampled(dir):
    """GPT-3 MLP fc2 shape (8 ranks, [256 x 6144] . [6144 x 12288] per step),
    add-and-forward hops, bf16 out: sampled rows against the oracle, and the
    whole output bitwise equal to the epilogue-add ring's."""
    N, m, k, n = 8, 256, 6144, 12288
    x_t, w_t = gen.rs_inputs_torch(N, m, k, n, "normal", 0, "cuda")
    ys = []
    for hop in ("add", "copy"):
        plan = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=1, out_dtype="bf16", n_comm=1,
                                hop=hop)
        y, ws = buffers.alloc_outputs(plan)
        say("hop full", dir, hop)
        buffers.run(plan, x_t, w_t, y, ws, comm=buffers.comm_streams(1))
        torch.cuda.synchronize()
        ys.append(y)
        del ws
    sampled_check("rs", N, m, x_t, w_t, ys[0], 8)
    assert torch.equal(ys[0], ys[1])
