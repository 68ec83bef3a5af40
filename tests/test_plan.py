"""Host logic: the ring planner's programs, simulated on the CPU.

Every program the library would enqueue is executed here in program order on
byte buffers (tests/ring_sim.py) with a happens-before race check, and its
result is compared with the oracle exactly (small-integer inputs, so every
fp32 sum is exact).  This covers, per the pages:
  * decomposed == monolithic, for every schedule, direction, chunk count and
    comm-stream count ("The idea" / "Why it works": linearity);
  * ring completeness: every AllGather output row-slice is written exactly
    once; every ReduceScatter bucket reaches its owner with all N
    contributions exactly once (rank-tagged powers of two);
  * ordering: no read before the producing copy or GEMM, no overwrite
    before the consumers are done (Megatron page, section 5), and a program
    with one dependency edge removed is caught;
  * the hop volume equals that of a ring AllGather / ReduceScatter.
"""
import itertools

import numpy as np
import pytest

import oracle
from collective_matmul_decomposition_amd import _native as nat
from collective_matmul_decomposition_amd import inputs as gen
from ring_sim import Race, Sim, buffer_sizes


def simulate(op, N, m, k, n, dir="uni", chunks=1, sched="decomposed", out="f32", n_comm=1, seed=0, dist="int",
             data=None, bucket="f32", hop="copy", group=0):
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, sched=sched, out_dtype=out,
                            n_comm=n_comm, bucket=bucket, hop=hop, group=group)
    if data is None:
        if op == "ag":
            a, w = gen.ag_inputs(N, m, k, n, dist, seed)
        else:
            a, w = gen.rs_inputs(N, m, k, n, dist, seed)
    else:
        a, w = data
    sizes = buffer_sizes(plan)
    sim = Sim(plan, sizes, {nat.CM_BUF_X: a, nat.CM_BUF_W: w}).run()
    return plan, sim, a, w


def output(sim, plan):
    d = plan.desc
    y = sim.buf[nat.CM_BUF_Y]
    if d.out_dtype == nat.CM_F32:
        return y.view(np.float32).astype(np.float64)
    return y.view(np.uint16)


def expect(op, a, w, out):
    ref = oracle.ag_gemm(a, w) if op == "ag" else oracle.gemm_rs(a, w)
    return ref.reshape(-1) if out == "f32" else oracle.round_bf16(ref).reshape(-1)


CASES = []
for N in (1, 2, 3, 4, 5, 8):
    for op, dir, sched, chunks in [("ag", "uni", "decomposed", 1), ("ag", "uni", "decomposed", 2),
                                   ("ag", "bi", "decomposed", 1), ("ag", "bi", "decomposed", 4),
                                   ("ag", "uni", "naive", 1),
                                   ("rs", "uni", "decomposed", 1), ("rs", "uni", "decomposed", 2),
                                   ("rs", "bi", "decomposed", 2), ("rs", "bi", "decomposed", 1),
                                   ("rs_pipe", "uni", "decomposed", 2), ("rs_pipe", "uni", "decomposed", 4),
                                   ("rs", "uni", "naive", 1),
                                   ("ag", "direct", "decomposed", 1), ("ag", "direct", "decomposed", 2),
                                   ("rs", "direct", "decomposed", 1), ("rs", "direct", "decomposed", 2)]:
        for n_comm in sorted({1, 2, 3, N, 2 * N}):
            CASES.append((op, N, dir, sched, chunks, n_comm))


BF16_BUCKET = [(N, dir, chunks, n_comm) for N in (1, 2, 3, 4, 5, 8) for dir in ("uni", "bi")
               for chunks in (1, 2) for n_comm in sorted({1, N})]


@pytest.mark.parametrize("N,dir,chunks,n_comm", BF16_BUCKET)
def test_bf16_bucket_program_matches_oracle(N, dir, chunks, n_comm):
    """The bf16-bucket RS program visits the ranks in the order the oracle's
    definition does: with integer data large enough that nearly every bucket
    addition rounds, the simulated result equals the oracle's bit for bit."""
    m, k, n = 3, 64, 64 * chunks
    rng = np.random.default_rng(100 + N)
    hv = rng.integers(-40, 41, (N, N * m, k)).astype(np.float32)
    wv = rng.integers(-40, 41, (N, n, k)).astype(np.float32)
    data = (gen.f32_to_bf16_bits(hv), gen.f32_to_bf16_bits(wv))
    plan, sim, a, w = simulate("rs", N, m, k, n, dir, chunks, "decomposed", "f32", n_comm, data=data, bucket="bf16")
    f32_plan = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, n_comm=n_comm)
    assert 2 * plan.ws_bytes == f32_plan.ws_bytes  # half the bucket bytes
    got = output(sim, plan)
    ref = oracle.gemm_rs_bf16_bucket(a, w, dir=dir).reshape(-1)
    assert np.array_equal(got, ref)
    if N > 2:  # rounding acted: the fp32-bucket result differs
        assert not np.array_equal(got, oracle.gemm_rs(a, w).reshape(-1))
    assert (sim.writes[nat.CM_BUF_Y] == 1).all()


HOP_ADD = [(N, dir, chunks, n_comm) for N in (1, 2, 3, 4, 5, 8) for dir in ("uni", "bi")
           for chunks in (1, 2) for n_comm in sorted({1, 2, N})]


@pytest.mark.parametrize("N,dir,chunks,n_comm", HOP_ADD)
def test_hop_add_program_matches_oracle_and_the_epilogue_ring(N, dir, chunks, n_comm):
    """Add-and-forward hops: exact on integers against the oracle, race-free,
    every output written once, and no copies (the adds are the hops).  That
    the GPU sums equal the epilogue-add ring's bitwise is a GPU test: this
    simulation adds in float64."""
    m, k, n = 3, 64, 64 * chunks
    for out in ("f32", "bf16"):
        plan, sim, a, w = simulate("rs", N, m, k, n, dir, chunks, "decomposed", out, n_comm, hop="add")
        assert np.array_equal(output(sim, plan), expect("rs", a, w, out))
        assert (sim.writes[nat.CM_BUF_Y] == 1).all()
    ops, _ = nat.cm_plan_program(nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks,
                                                  n_comm=n_comm, hop="add"))
    assert not any(o.kind == nat.CM_OPK_COPY for o in ops)


@pytest.mark.parametrize("N", [3, 4, 8])
def test_hop_add_gemms_do_not_wait_for_the_previous_hop(N):
    """With add-and-forward hops the GEMM of step s waits only for the add of
    step s - 2 (its partial slot's last reader), never for hop(s - 1); the
    owner's last GEMM waits for the last add."""
    plan = nat.cm_ring_plan(op="rs", n_ranks=N, m=8, k=64, n=128, chunks=1, n_comm=1, hop="add", group=1)
    ops, _ = nat.cm_plan_program(plan)
    recorded_at = {}
    for o in ops:
        if o.kind == nat.CM_OPK_RECORD and o.stream != 0:
            recorded_at[o.event] = o.step
    for o in ops:
        if o.kind == nat.CM_OPK_WAIT and o.stream == 0 and 0 <= o.step < N - 1:
            assert recorded_at[o.event] <= o.step - 2, (o.step, recorded_at[o.event])
    last_waits = [recorded_at[o.event] for o in ops if o.kind == nat.CM_OPK_WAIT and o.stream == 0
                  and o.step == N - 1]
    assert last_waits == [N - 2]


@pytest.mark.parametrize("dir,chunks,n_comm", [("uni", 1, 1), ("uni", 2, 2), ("bi", 1, 2), ("direct", 1, 1)])
def test_ag_step0_gemm_is_emitted_before_the_hops(dir, chunks, n_comm):
    """A graph dispatches nodes in program order: step 0's GEMM, which reads
    only the ranks' own shards, comes before step 0's hop copies of the same
    chunk (emitted after them, it started behind the copies)."""
    plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=16, k=64, n=64, dir=dir, chunks=chunks, n_comm=n_comm, group=1)
    ops, jobs = nat.cm_plan_program(plan)
    for j in range(plan.chunks):
        idx = [i for i, o in enumerate(ops) if o.step == 0 and o.chunk == j and o.kind in (nat.CM_OPK_GEMM,
                                                                                          nat.CM_OPK_COPY)]
        kinds = [ops[i].kind for i in idx]
        assert kinds[0] == nat.CM_OPK_GEMM and nat.CM_OPK_COPY in kinds, kinds
        g = ops[idx[0]]
        assert all(jb.a_buf == nat.CM_BUF_X for jb in jobs[g.first_job:g.first_job + g.n_jobs])


@pytest.mark.parametrize("op", ["ag", "rs"])
def test_share_step_gemm_is_emitted_before_its_hop(op):
    """One rank's share: every step's GEMM precedes that step's hop in program
    order (the hop does not depend on it)."""
    plan = nat.cm_ring_plan(op=op, n_ranks=5, m=16, k=256, n=64, share=1, split_k=2)
    ops, _ = nat.cm_plan_program(plan)
    for s in range(4):
        first = [o.kind for o in ops if o.step == s and o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_COPY)]
        assert first == [nat.CM_OPK_GEMM, nat.CM_OPK_COPY], (s, first)


PIPE_ADD = [(N, chunks, n_comm, sched) for N in (1, 2, 3, 4, 5, 8) for chunks in (1, 2, 4)
            for n_comm in sorted({1, 2, N}) for sched in ("decomposed", "naive") if sched == "decomposed" or chunks == 1]


@pytest.mark.parametrize("N,chunks,n_comm,sched", PIPE_ADD)
def test_pipe_hop_add_program_matches_oracle(N, chunks, n_comm, sched):
    """Pipeline-chunk (and naive) ReduceScatter with add-and-forward hops:
    exact on integers against the oracle, race-free, each output written once,
    no copies, and no GEMM waits for a comm stream (every chunk has its own
    ring slots)."""
    m, k, n = 3, 64, 64 * chunks
    op = "rs_pipe" if sched == "decomposed" else "rs"
    for out in ("f32", "bf16"):
        plan, sim, a, w = simulate(op, N, m, k, n, "uni", chunks, sched, out, n_comm, hop="add")
        assert np.array_equal(output(sim, plan), expect("rs", a, w, out))
        assert (sim.writes[nat.CM_BUF_Y] == 1).all()
    ops, _ = nat.cm_plan_program(plan)
    assert not any(o.kind == nat.CM_OPK_COPY for o in ops)
    assert not any(o.kind == nat.CM_OPK_WAIT and o.stream == 0 and o.step >= 0 for o in ops)


def test_pipe_hop_add_splits_large_launches():
    # N = 16: 256 (rank, bucket) jobs per chunk in launches of at most 128
    plan, sim, a, w = simulate("rs_pipe", 16, 2, 64, 128, "uni", 2, "decomposed", "f32", 1, hop="add")
    assert np.array_equal(output(sim, plan), expect("rs", a, w, "f32"))
    ops, _ = nat.cm_plan_program(plan)
    assert max(o.n_jobs for o in ops if o.kind == nat.CM_OPK_GEMM) <= 128


def test_hop_add_is_only_for_the_ring_rs():
    base = dict(n_ranks=4, m=8, k=64, n=128, hop="add")
    for kw in (dict(op="ag"), dict(op="rs", dir="direct"), dict(op="rs", bucket="bf16")):
        st, _ = nat.cm_ring_plan_status(nat.make_desc(**dict(base, **kw)))
        assert st == nat.CM_ERR_UNSUPPORTED, kw
    st, _ = nat.cm_ring_plan_status(nat.make_desc(op="rs", n_ranks=4, m=8, k=64, n=128, hop=2))
    assert st == nat.CM_ERR_INVALID_ARG
    p = nat.cm_ring_plan(op="rs", n_ranks=4, m=8, k=64, n=128, sched="auto", hop="add", copy_gbps=1.0)
    assert p.desc.sched in (nat.CM_SCHED_DECOMPOSED, nat.CM_SCHED_NAIVE)


def test_auto_schedule_declines_when_hops_cannot_hide():
    """The decline gate of the decomposition page: the cost model keeps the
    decomposed op where it predicts a win and falls back to the naive
    schedule where the hops are longer than the compute."""
    big = dict(n_ranks=8, m=256, k=12288, n=6144, n_comm=1)
    p = nat.cm_ring_plan(op="ag", sched="auto", **big)
    assert p.desc.sched == nat.CM_SCHED_DECOMPOSED and p.declined == 0
    # thin compute, same hops: the rewrite is declined
    thin = dict(n_ranks=8, m=256, k=12288, n=64, n_comm=1, copy_gbps=20.0)
    p = nat.cm_ring_plan(op="ag", sched="auto", **thin)
    assert p.desc.sched == nat.CM_SCHED_NAIVE and p.declined == 1
    naive = nat.cm_ring_plan(op="ag", sched="naive", **thin)
    dec = nat.cm_ring_plan(op="ag", sched="decomposed", **thin)
    assert naive.est_total_us < dec.est_total_us
    # the resolved plan runs like an explicit one
    plan, sim, a, w = None, None, None, None
    for op in ("ag", "rs"):
        for kw in (dict(n_ranks=4, m=8, k=64, n=64, copy_gbps=1.0), dict(n_ranks=4, m=8, k=64, n=64)):
            pl = nat.cm_ring_plan(op=op, sched="auto", **kw)
            ref = nat.cm_ring_plan(op=op, sched=pl.desc.sched, chunks=pl.chunks, **kw)
            assert (pl.n_ops, pl.n_jobs, pl.ws_bytes) == (ref.n_ops, ref.n_jobs, ref.ws_bytes)


def test_direct_schedules_fetch_from_owners():
    """AG direct: every hop copies from the user's input (owner -> consumer);
    RS direct: every partial goes to its owner, whose adds follow the ring order."""
    p = nat.cm_ring_plan(op="ag", n_ranks=6, m=8, k=64, n=64, dir="direct", n_comm=2)
    ops, _ = nat.cm_plan_program(p)
    copies = [o for o in ops if o.kind == nat.CM_OPK_COPY]
    assert copies and all(o.src_buf == nat.CM_BUF_X and o.dst_buf == nat.CM_BUF_WS for o in copies)
    assert sum(o.bytes for o in copies) == 6 * 5 * 8 * 64 * 2  # the ring AllGather volume
    p = nat.cm_ring_plan(op="rs", n_ranks=6, m=8, k=64, n=128, dir="direct", n_comm=2)
    ops, _ = nat.cm_plan_program(p)
    copies = [o for o in ops if o.kind == nat.CM_OPK_COPY]
    assert sum(o.bytes for o in copies) == 6 * 5 * 8 * 128 * 4  # the ring ReduceScatter volume
    assert sum(1 for o in ops if o.kind == nat.CM_OPK_REDUCE) == p.chunks * (6 - 2)  # one add per step and chunk


def test_pick_one_of_two_collectives():
    """An einsum with a gathered input and a reduce-scattered output overlaps
    only one of them: the cost model picks the candidate with the larger
    predicted saving (naive minus decomposed time), or neither."""
    # the AllGather side has shard hops and a wide GEMM to hide them; the
    # ReduceScatter side moves 64-column buckets, with little to hide
    ag = dict(op="ag", n_ranks=8, m=256, k=8192, n=8192, n_comm=1)
    rs = dict(op="rs", n_ranks=8, m=256, k=8192, n=64, n_comm=1)
    choice, (s_ag, s_rs) = nat.cm_pick_overlap(ag, rs)
    assert choice == 0 and s_ag > 0 > s_rs
    # the other way round
    choice, (s_ag, s_rs) = nat.cm_pick_overlap(dict(ag, k=64, n=64), dict(rs, n=8192))
    assert choice == 1 and s_rs > 0 > s_ag
    # links too slow for either to hide: neither
    choice, (s_ag, s_rs) = nat.cm_pick_overlap(dict(ag, copy_gbps=0.5, k=64, n=64),
                                               dict(rs, copy_gbps=0.5, k=64, n=64))
    assert choice == -1 and s_ag <= 0 and s_rs <= 0
    # the savings are the gate's own estimates
    for d in (ag, dict(rs, n=8192)):
        dec = nat.cm_ring_plan(sched="decomposed", **d)
        nai = nat.cm_ring_plan(sched="naive", **d)
        _, sv = nat.cm_pick_overlap(d if d["op"] == "ag" else ag, d if d["op"] == "rs" else rs)
        assert abs(sv[0 if d["op"] == "ag" else 1] - (nai.est_total_us - dec.est_total_us)) < 1e-6
    with pytest.raises(nat.CMError):
        nat.cm_pick_overlap(rs, ag)


def test_bf16_bucket_is_only_for_the_decomposed_rs():
    for kw in (dict(op="ag"), dict(op="rs_pipe", chunks=2), dict(op="rs", sched="naive")):
        st, _ = nat.cm_ring_plan_status(nat.make_desc(**dict(dict(n_ranks=4, m=8, k=64, n=128, bucket="bf16"), **kw)))
        assert st == nat.CM_ERR_UNSUPPORTED


@pytest.mark.parametrize("op,N,dir,sched,chunks,n_comm", CASES)
def test_program_matches_oracle_and_is_race_free(op, N, dir, sched, chunks, n_comm):
    m = 4 * chunks if op == "ag" else 3
    k = 64
    n = 64 * chunks if op != "ag" else 64
    for out in ("f32", "bf16"):
        plan, sim, a, w = simulate(op, N, m, k, n, dir, chunks, sched, out, n_comm)
        got = output(sim, plan)
        assert np.array_equal(got, expect(op, a, w, out)), (op, N, dir, sched, chunks, n_comm, out)
        # every output element is written exactly once
        assert (sim.writes[nat.CM_BUF_Y] == 1).all()


@pytest.mark.parametrize("op,dir,chunks", [("rs", "uni", 1), ("rs", "bi", 2), ("rs_pipe", "uni", 2),
                                           ("rs", "uni", 4)])
@pytest.mark.parametrize("N", [2, 3, 5, 8])
def test_every_bucket_collects_every_rank_once(op, dir, chunks, N):
    """H_r = 2^r everywhere and W_r = identity: Out_q must be 2^N - 1 (each rank once)."""
    m, k = 2, 64 * chunks
    n = k
    h = np.stack([np.full((N * m, k), 2.0 ** r, np.float32) for r in range(N)])
    w = np.stack([np.eye(k, dtype=np.float32)] * N)
    plan, sim, _, _ = simulate(op, N, m, k, n, dir, chunks, "decomposed", "f32", N,
                               data=(gen.f32_to_bf16_bits(h), gen.f32_to_bf16_bits(w)))
    got = output(sim, plan).reshape(N, m, n)
    assert (got == 2.0 ** N - 1).all()


@pytest.mark.parametrize("dir", ["uni", "bi"])
@pytest.mark.parametrize("N", [3, 4, 7, 8])
def test_allgather_uses_every_shard_once(dir, N):
    """Each Y_r row block c is written by exactly one job, and that job multiplied shard c."""
    plan = nat.cm_ring_plan(op="ag", n_ranks=N, m=8, k=64, n=64, dir=dir, chunks=2, n_comm=2)
    ops, jobs = nat.cm_plan_program(plan)
    seen = {}
    for o in ops:
        if o.kind != nat.CM_OPK_GEMM:
            continue
        for j in jobs[o.first_job:o.first_job + o.n_jobs]:
            key = (j.rank, j.index, o.chunk)
            assert key not in seen
            seen[key] = o.step
            # the output rows are shard `index`'s rows of Y_rank
            row = (j.c_off // (64 * 2)) - j.rank * N * 8
            assert row == j.index * 8 + o.chunk * 4
    assert len(seen) == N * N * 2
    # compute steps: N (uni) or 1 + ceil((N-1)/2) (bi)
    assert plan.n_steps == (N if dir == "uni" else 1 + (N - 1 + 1) // 2)
    assert plan.arc_cw + plan.arc_ccw == N - 1


@pytest.mark.parametrize("op", ["ag", "rs", "rs_pipe"])
@pytest.mark.parametrize("dir", ["uni", "bi"])
@pytest.mark.parametrize("N", [2, 4, 8])
def test_hop_volume_is_the_ring_volume(op, dir, N):
    """Total hop bytes = N (N - 1) shard (AG, bf16) or bucket (RS, fp32) sizes."""
    m, k, n = 8, 128, 256
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=2, n_comm=4)
    ops, _ = nat.cm_plan_program(plan)
    total = sum(o.bytes for o in ops if o.kind == nat.CM_OPK_COPY)
    per = m * k * 2 if op == "ag" else m * n * 4
    assert total == N * (N - 1) * per


@pytest.mark.parametrize("op,dir,group", [("ag", "uni", 0), ("ag", "uni", 1), ("ag", "bi", 0), ("ag", "bi", 1),
                                          ("rs", "uni", 0), ("rs", "bi", 0)])
@pytest.mark.parametrize("n_comm", [1, 2, 3])
def test_every_hop_is_one_copy_per_lane(op, dir, group, n_comm):
    """Receive slots are indexed by shard (AG) or bucket (copy-hop RS), so a
    hop moves a lane's range in place: one contiguous copy per lane, never
    split at the ring's wrap-around (shard-sized copies only at an AllGather's
    first hop with several chunks per shard, not used here)."""
    N, m, k, n = 8, 16, 128, 256
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=1, n_comm=n_comm, group=group)
    ops, _ = nat.cm_plan_program(plan)
    copies = [o for o in ops if o.kind == nat.CM_OPK_COPY]
    per_hop = {}
    for o in copies:
        per_hop.setdefault((o.step, o.chunk, o.stream), []).append(o)
    # one copy per (step, lane, direction) and each covers a whole lane range of
    # shards or buckets; with one lane the two directions share it
    lanes = min(n_comm, 3)
    ndir = 2 if dir == "bi" else 1
    per_lane = ndir if lanes < ndir else 1
    assert all(len(v) <= per_lane for v in per_hop.values()), {key: len(v) for key, v in per_hop.items()}
    blk = m * k * 2 if op == "ag" else m * n * 4
    assert all(o.bytes % blk == 0 and o.bytes >= blk for o in copies)
    assert max(o.bytes for o in copies) <= blk * -(-N // max(1, lanes // ndir))


def _drop_op(sim, index):
    sim.ops = sim.ops[:index] + sim.ops[index + 1:]
    return sim


@pytest.mark.parametrize("op,dir,chunks,hop", [("ag", "uni", 1, "copy"), ("ag", "bi", 2, "copy"),
                                               ("rs", "uni", 2, "copy"), ("rs", "bi", 2, "copy"),
                                               ("rs_pipe", "uni", 2, "copy"), ("ag", "uni", 2, "copy"),
                                               ("rs", "uni", 1, "add"), ("rs", "bi", 2, "add"),
                                               ("rs_pipe", "uni", 2, "add")])
def test_dropped_dependency_is_caught(op, dir, chunks, hop):
    """Negative control: removing any one wait that orders a hop against a GEMM makes a race."""
    N, m, k = 4, 4 * chunks, 64
    n = 64 * chunks
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m if op == "ag" else 3, k=k, n=n if op != "ag" else 64, dir=dir,
                            chunks=chunks, n_comm=2, hop=hop)
    sizes = buffer_sizes(plan)
    if op == "ag":
        a, w = gen.ag_inputs(N, plan.desc.m, k, plan.desc.n, "int", 0)
    else:
        a, w = gen.rs_inputs(N, plan.desc.m, k, plan.desc.n, "int", 0)
    base = Sim(plan, sizes, {nat.CM_BUF_X: a, nat.CM_BUF_W: w})
    waits = [i for i, o in enumerate(base.ops) if o.kind == nat.CM_OPK_WAIT and o.step >= 0]
    assert waits
    caught = 0
    for i in waits:
        sim = _drop_op(Sim(plan, sizes, {nat.CM_BUF_X: a, nat.CM_BUF_W: w}), i)
        try:
            sim.run()
        except Race:
            caught += 1
    # every in-schedule wait is load-bearing
    assert caught == len(waits), "%d of %d dropped waits went unnoticed" % (len(waits) - caught, len(waits))


def test_entry_and_exit_edges_are_needed():
    plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=4, k=64, n=64, n_comm=2)
    sizes = buffer_sizes(plan)
    a, w = gen.ag_inputs(4, 4, 64, 64, "int", 0)
    ops = Sim(plan, sizes).ops
    exit_waits = [i for i, o in enumerate(ops) if o.kind == nat.CM_OPK_WAIT and o.step < 0 and o.stream == 0]
    entry_waits = [i for i, o in enumerate(ops) if o.kind == nat.CM_OPK_WAIT and o.step < 0 and o.stream != 0]
    for i in exit_waits + entry_waits:
        sim = _drop_op(Sim(plan, sizes, {nat.CM_BUF_X: a, nat.CM_BUF_W: w}), i)
        with pytest.raises(Race):
            sim.run()


def _gpu_cases():
    import test_gpu_parity as g
    cases = []
    for op, dir, sched, chunks, dist, out in g.TINY:
        cases.append(dict(op=op, n_ranks=4, m=64, k=256, n=256, dir=dir, chunks=chunks, sched=sched, out_dtype=out,
                          n_comm=4))
    for op, N, m, k, n, dir, chunks, n_comm in g.RAGGED:
        for out in ("f32", "bf16"):
            cases.append(dict(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype=out, n_comm=n_comm))
    for op, dir, chunks in g.MID:
        k, n = (1024, 768) if op == "ag" else (768, 1024)
        cases.append(dict(op=op, n_ranks=8, m=256, k=k, n=n, dir=dir, chunks=chunks, out_dtype="f32", n_comm=8))
    for op, N, m, k, n, dir, n_comm, chunks in g.FULL:
        cases.append(dict(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype="bf16", n_comm=n_comm))
    for op, N, c in g.C4:
        k, n = (2048, 8192 // N) if op == "ag" else (8192 // N, 2048)
        cases.append(dict(op=op, n_ranks=N, m=1024 // N, k=k, n=n, chunks=c, out_dtype="f32", n_comm=1))
    for op, k, n, chunks in g.C5:
        cases.append(dict(op=op, n_ranks=8, m=512, k=k, n=n, chunks=chunks, out_dtype="bf16", n_comm=1))
    for N, m, k, n, dir, chunks, out in g.BF16B:
        cases.append(dict(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype=out, n_comm=2,
                          bucket="bf16"))
    cases.append(dict(op="rs", n_ranks=8, m=256, k=6144, n=12288, chunks=1, out_dtype="bf16", n_comm=1, bucket="bf16"))
    for op, N, m, k, n, chunks, n_comm in g.DIRECT:
        cases.append(dict(op=op, n_ranks=N, m=m, k=k, n=n, dir="direct", chunks=chunks, out_dtype="f32", n_comm=n_comm))
    cases.append(dict(op="ag", n_ranks=8, m=256, k=12288, n=6144, dir="direct", chunks=1, out_dtype="bf16", n_comm=1))
    cases.append(dict(op="rs", n_ranks=8, m=256, k=6144, n=12288, dir="direct", chunks=1, out_dtype="bf16", n_comm=1))
    for N, m, k, n, dir, chunks, n_comm in g.HOP_ADD:
        for out in ("f32", "bf16"):
            cases.append(dict(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype=out,
                              n_comm=n_comm, hop="add"))
    for dir in ("uni", "bi"):
        cases.append(dict(op="rs", n_ranks=8, m=256, k=6144, n=12288, dir=dir, chunks=1, out_dtype="bf16", n_comm=1,
                          hop="add"))
    for op, N, m, k, n, chunks, n_comm, sched in g.PIPE_ADD:
        for out in ("f32", "bf16"):
            cases.append(dict(op=op, n_ranks=N, m=m, k=k, n=n, chunks=chunks, out_dtype=out, n_comm=n_comm,
                              sched=sched, hop="add"))
    for hop in ("add", "copy"):
        cases.append(dict(op="rs_pipe", n_ranks=8, m=512, k=1024, n=8192, chunks=4, out_dtype="f32", n_comm=1, hop=hop))
    for op in ("ag", "rs", "rs_pipe"):
        for kw in (dict(), dict(copy_gbps=1.0)):
            cases.append(dict(op=op, n_ranks=4, m=64, k=256, n=256, sched="auto", out_dtype="f32", n_comm=2, **kw))
    for tile in g.TILES:
        for op in ("ag", "rs"):
            for out in ("f32", "bf16"):
                cases.append(dict(op=op, n_ranks=3, m=300, k=192, n=320 if op == "ag" else 640, n_comm=2,
                                  chunks=1 if op == "ag" else 2, out_dtype=out, tile=tile))
    for op, N, m, k, n, dir, chunks, n_comm, hop in g.EXTREME:
        for out in ("f32", "bf16"):
            cases.append(dict(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype=out, n_comm=n_comm,
                              hop=hop))
    return cases


@pytest.mark.parametrize("case", range(11))
def test_extreme_programs_simulate(case):
    """The limits the GPU tests run (64 virtual ranks with 1-3 rows per shard on every
    schedule; 16 chunks), executed on the CPU with the race check: equal to the oracle."""
    import test_gpu_parity as g
    op, N, m, k, n, dir, chunks, n_comm, hop = g.EXTREME[case]
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype="f32", n_comm=n_comm,
                            hop=hop)
    a, w = (gen.ag_inputs if op == "ag" else gen.rs_inputs)(N, m, k, n, "int", 0)
    sim = Sim(plan, buffer_sizes(plan), {nat.CM_BUF_X: a, nat.CM_BUF_W: w}).run()
    ref = oracle.ag_gemm(a, w) if op == "ag" else oracle.gemm_rs(a, w)
    got = sim.buf[nat.CM_BUF_Y].view(np.float32).reshape(ref.shape).astype(np.float64)
    assert np.array_equal(got, ref)


def test_gpu_test_programs_stay_in_bounds():
    """Every program the GPU tests launch is checked on the CPU first: in-bounds, aligned, <= 128 jobs."""
    from ring_sim import check_program_bounds
    for kw in _gpu_cases():
        plan = nat.cm_ring_plan(**kw)
        check_program_bounds(plan)


# ------------------------------------------------------------ measurement modes and lanes
@pytest.mark.parametrize("op,dir,hop", [("ag", "uni", "copy"), ("ag", "bi", "copy"), ("rs", "uni", "add"),
                                        ("rs", "bi", "copy"), ("rs_pipe", "uni", "add")])
@pytest.mark.parametrize("skip", ["hops", "gemms"])
def test_skip_modes_keep_the_program(op, dir, hop, skip):
    """The G-alone / C-alone modes run the same program (same launches, copies
    and ordering edges); the executor only empties one class of operations."""
    kw = dict(op=op, n_ranks=5, m=32, k=128, n=256, dir=dir, chunks=2, out_dtype="f32", n_comm=2,
              hop=hop if op != "ag" else "copy")
    base = nat.cm_ring_plan(**kw)
    meas = nat.cm_ring_plan(skip=skip, **kw)
    assert meas.desc.skip == nat._ENUMS["skip"][skip]
    ops0, jobs0 = nat.cm_plan_program(base)
    ops1, jobs1 = nat.cm_plan_program(meas)
    key = lambda o: (o.kind, o.stream, o.event, o.step, o.chunk, o.first_job, o.n_jobs, o.rows, o.cols, o.depth,
                     o.src_buf, o.dst_buf, o.src_off, o.dst_off, o.bytes)
    assert [key(o) for o in ops0] == [key(o) for o in ops1]
    assert (base.n_ops, base.n_jobs, base.n_events, base.ws_bytes) == (meas.n_ops, meas.n_jobs, meas.n_events,
                                                                      meas.ws_bytes)
    # each mode empties something, and not everything
    hops = [o for o in ops1 if o.kind == nat.CM_OPK_COPY or (o.kind == nat.CM_OPK_REDUCE and o.stream != 0)]
    gemms = [o for o in ops1 if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_REDUCE) and o.stream == 0]
    assert hops and gemms


def test_unknown_skip_mode_is_rejected():
    st, _ = nat.cm_ring_plan_status(nat.make_desc("ag", 4, 16, 64, 64, skip=3))
    assert st == nat.CM_ERR_INVALID_ARG
    st, _ = nat.cm_ring_plan_status(nat.make_desc("allgather", 4, 16, 64, 0, skip=-1))
    assert st == nat.CM_ERR_INVALID_ARG


@pytest.mark.parametrize("op,dir", [("ag", "uni"), ("ag", "bi"), ("rs", "uni"), ("rs", "bi"), ("rs", "direct"),
                                    ("rs_pipe", "uni")])
@pytest.mark.parametrize("n_comm", [4, 8, 16])
def test_programs_use_at_most_three_comm_lanes(op, dir, n_comm):
    """A process has four hardware queues by default: the compute stream plus at
    most three comm lanes run side by side.  Streams beyond three are accepted
    and left idle, and the program still equals the oracle."""
    plan, sim, a, w = simulate(op, 8, 16, 128, 256, dir=dir, chunks=2, n_comm=n_comm)
    ops, _ = nat.cm_plan_program(plan)
    work = {o.stream for o in ops if o.kind in (nat.CM_OPK_COPY, nat.CM_OPK_REDUCE, nat.CM_OPK_GEMM)}
    assert max(work) <= 3
    assert np.array_equal(output(sim, plan), expect("ag" if op == "ag" else "rs", a, w, "f32"))


def test_stress_mode_is_eager_only():
    """The race-stress test mode exists in the eager executor only; it does not
    change the program."""
    st, _ = nat.cm_ring_plan_status(nat.make_desc("ag", 4, 64, 256, 256, stress=1))
    assert st == nat.CM_ERR_UNSUPPORTED
    a = nat.cm_ring_plan(op="rs", n_ranks=4, m=64, k=256, n=256, chunks=2, exec_mode="eager", stress=7)
    b = nat.cm_ring_plan(op="rs", n_ranks=4, m=64, k=256, n=256, chunks=2, exec_mode="eager")
    assert (a.n_ops, a.n_jobs, a.n_events, a.ws_bytes) == (b.n_ops, b.n_jobs, b.n_events, b.ws_bytes)


# ---------------------------------------------------------------- grouped launches
GROUPED = [(op, N, dir, g, n_comm) for op in ("ag", "rs") for N in (2, 3, 4, 5, 8) for dir in ("uni", "bi")
           for g in (2, 3, 4) for n_comm in sorted({1, 2, N})]


def _partition(plan):
    return list(plan.group_len[:plan.n_launches])


@pytest.mark.parametrize("op,N,dir,g,n_comm", GROUPED)
def test_grouped_launches_match_oracle(op, N, dir, g, n_comm):
    """Steps grouped per launch (at most g): exact on integers against the
    oracle, race-free, every output written once; the launch partition
    covers every step once, the ReduceScatter's owner step is a launch of its
    own, and each launch's jobs come in runs of b_share that read the same
    weights."""
    m, k, n = 3, 64, 64
    hop = "add" if op == "rs" else "copy"
    for out in ("f32", "bf16"):
        plan, sim, a, w = simulate(op, N, m, k, n, dir, 1, "decomposed", out, n_comm, hop=hop, group=g)
        assert np.array_equal(output(sim, plan), expect(op, a, w, out))
        assert (sim.writes[nat.CM_BUF_Y] == 1).all()
    part = _partition(plan)
    assert sum(part) == plan.n_steps and all(1 <= x <= g for x in part)
    ops, jobs = nat.cm_plan_program(plan)
    if op == "rs" and any(x > 1 for x in part):
        # the owners' final add on a comm stream writes the output, after every other op of the call
        writers = [o for o in ops if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_REDUCE)
                   and any(j.c_buf == nat.CM_BUF_Y for j in jobs[o.first_job:o.first_job + o.n_jobs])]
        assert len(writers) == 1 and writers[0].kind == nat.CM_OPK_REDUCE and writers[0].stream != 0
        # bidirectional: both arrivals; one-way with N >= 3: the last hop's bucket and partial (fused add)
        assert writers[0].depth == (2 if N > 2 else 1)
    gemms = [o for o in ops if o.kind == nat.CM_OPK_GEMM]
    assert len(gemms) == plan.n_launches
    for o in gemms:
        assert o.b_share >= 1 and o.n_jobs % o.b_share == 0 and o.n_jobs <= 128
        js = jobs[o.first_job:o.first_job + o.n_jobs]
        for i in range(0, o.n_jobs, o.b_share):
            run = js[i:i + o.b_share]
            assert len({(j.b_buf, j.b_off, j.rank) for j in run}) == 1
    if any(x > 1 for x in part):
        assert plan.slots == (max(2, plan.arc_cw) if op == "ag" else max(2, plan.n_steps))


@pytest.mark.parametrize("op,N", [("ag", 8), ("rs", 8)])
def test_group_one_is_the_step_program(op, N):
    """group = 1 is the one-step-per-launch program; every group setting
    multiplies the same shards into the same outputs."""
    hop = "add" if op == "rs" else "copy"
    kw = dict(op=op, n_ranks=N, m=4, k=64, n=64, chunks=1, n_comm=1, hop=hop)
    p1 = nat.cm_ring_plan(group=1, **kw)
    assert _partition(p1) == [1] * p1.n_steps and p1.slots == 2
    ops1, jobs1 = nat.cm_plan_program(p1)
    assert all(o.b_share == 1 for o in ops1 if o.kind == nat.CM_OPK_GEMM)
    key = lambda j: (j.rank, j.dir, j.index)
    for g in (2, 3, 4):
        pg = nat.cm_ring_plan(group=g, **kw)
        _, jobsg = nat.cm_plan_program(pg)
        gem1 = sorted(key(j) for j in jobs1 if j.a_buf >= 0)
        gemg = sorted(key(j) for j in jobsg if j.a_buf >= 0)
        assert gem1 == gemg


@pytest.mark.parametrize("op,dir", [("ag", "uni"), ("ag", "bi"), ("rs", "uni"), ("rs", "bi")])
def test_grouped_dropped_dependency_is_caught(op, dir):
    """Negative control for grouped launches: removing any one in-schedule wait makes a race."""
    N, m, k, n = 5, 3, 64, 64
    hop = "add" if op == "rs" else "copy"
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=1, n_comm=2, hop=hop, group=2)
    assert any(x > 1 for x in _partition(plan))
    sizes = buffer_sizes(plan)
    a, w = (gen.ag_inputs if op == "ag" else gen.rs_inputs)(N, m, k, n, "int", 0)
    base = Sim(plan, sizes, {nat.CM_BUF_X: a, nat.CM_BUF_W: w})
    waits = [i for i, o in enumerate(base.ops) if o.kind == nat.CM_OPK_WAIT and o.step >= 0]
    assert waits
    caught = 0
    for i in waits:
        sim = _drop_op(Sim(plan, sizes, {nat.CM_BUF_X: a, nat.CM_BUF_W: w}), i)
        try:
            sim.run()
        except Race:
            caught += 1
    assert caught == len(waits), "%d of %d dropped waits went unnoticed" % (len(waits) - caught, len(waits))


def test_auto_groups_the_gpt3_step():
    """At the GPT-3 MLP shape the cost model groups steps (each rank's 151 MB
    of weights is then streamed once per launch instead of once per step)."""
    ag = nat.cm_ring_plan(op="ag", n_ranks=8, m=256, k=12288, n=6144, chunks=1, n_comm=1)
    rs = nat.cm_ring_plan(op="rs", n_ranks=8, m=256, k=6144, n=12288, chunks=1, n_comm=1, hop="add")
    for p in (ag, rs):
        assert p.n_launches < p.n_steps and sum(_partition(p)) == p.n_steps


REPLAN = [dict(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, n_comm=nc, hop=hop, group=g, copy_gbps=cg)
          for op, hop in (("ag", "copy"), ("rs", "add"), ("rs", "copy"), ("rs_pipe", "add"))
          for N, m, k, n in ((8, 256, 12288, 6144), (8, 512, 4096, 1792), (4, 16, 64, 64), (5, 3, 64, 128))
          for dir in ("uni", "bi") for nc in (1, 2) for g in (0, 2) for cg in (0.0, 333.0)
          if not (op == "rs_pipe" and dir == "bi")]


@pytest.mark.parametrize("kw", REPLAN)
def test_replanning_a_plans_request_reproduces_it(kw):
    """The executors re-derive a caller's plan from its own request (with its
    chunk count) and refuse a mismatch; planning must therefore be a fixed
    point: the filled-in request plans to the same schedule."""
    if kw["op"] == "ag":
        kw = dict(kw, n=kw["n"], k=kw["k"])
    else:
        kw = dict(kw, k=kw["n"] if kw["op"] == "ag" else kw["k"])
    p = nat.cm_ring_plan(**kw)
    d = nat.cm_plan_desc.from_buffer_copy(p.desc)
    d.chunks = p.chunks
    q = nat.cm_ring_plan(desc=d)
    for f in ("chunks", "n_steps", "arc_cw", "arc_ccw", "tile_m", "tile_n", "n_ops", "n_jobs", "n_events",
              "ws_bytes", "split", "n_launches", "slots"):
        assert getattr(p, f) == getattr(q, f), f
    assert list(p.group_len) == list(q.group_len)


ENGINE_CASES = [
    # GPT-3 MLP fc1: seven 50 MB SDMA hop steps hide under the step GEMMs
    (dict(op="ag", n_ranks=8, m=256, k=12288, n=6144), "sdma"),
    # add-and-forward hops copy nothing: the engines tie and SDMA is kept
    (dict(op="rs", n_ranks=8, m=256, k=6144, n=12288, hop="add"), "sdma"),
    # SP layer AllGather->QKV and ->fc1: the SDMA hop chain (67 MB a step) outlasts the GEMMs
    (dict(op="ag", n_ranks=8, m=512, k=8192, n=3072), "cu"),
    (dict(op="ag", n_ranks=8, m=512, k=8192, n=3584), "cu"),
]


def _plan_fields(p):
    return ([getattr(p, f) for f in ("chunks", "n_steps", "arc_cw", "arc_ccw", "tile_m", "tile_n", "n_ops", "n_jobs",
                                    "n_events", "ws_bytes", "split", "n_launches", "slots", "est_total_us")]
            + list(p.group_len))


@pytest.mark.parametrize("kw,engine", ENGINE_CASES)
def test_auto_copy_engine_picks_and_is_a_fixed_point(kw, engine):
    """copy_engine=auto plans the request with each engine and keeps one; the
    plan is the explicit engine's plan, its request names that engine, and
    re-planning that request reproduces it."""
    p = nat.cm_ring_plan(chunks=1, n_comm=1, copy_engine="auto", **kw)
    assert p.desc.copy_engine == nat._ENUMS["copy"][engine]
    q = nat.cm_ring_plan(chunks=1, n_comm=1, copy_engine=engine, **kw)
    assert _plan_fields(p) == _plan_fields(q)
    d = nat.cm_plan_desc.from_buffer_copy(p.desc)
    r = nat.cm_ring_plan(desc=d)
    assert _plan_fields(r) == _plan_fields(p) and r.desc.copy_engine == p.desc.copy_engine


def test_auto_copy_engine_in_the_layer_plan():
    """The SP layer's stages resolve the engine one by one: the AllGather
    stages whose SDMA hops would outlast the GEMMs take the copy kernel, the
    add-and-forward ReduceScatters keep SDMA; re-planning the layer's request
    gives the same stage plans."""
    lp = nat.cm_plan_layer(n_ranks=8, m=512, d=8192, heads=8, ffn=3584, n_comm=1, copy_engine="auto",
                           ag_chunks=1, rs_chunks=1)
    eng = {s: getattr(lp, s).desc.copy_engine for s in ("qkv", "proj", "fc1", "fc2")}
    assert eng == {"qkv": nat.CM_COPY_CU, "proj": nat.CM_COPY_SDMA, "fc1": nat.CM_COPY_CU, "fc2": nat.CM_COPY_SDMA}
    assert lp.desc.copy_engine == nat.CM_COPY_AUTO
    again = nat.cm_plan_layer(desc=nat.cm_layer_desc.from_buffer_copy(lp.desc))
    for s in ("qkv", "proj", "fc1", "fc2"):
        assert _plan_fields(getattr(again, s)) == _plan_fields(getattr(lp, s))
