"""One rank's share (cm_plan_desc.share = 1), on the CPU: validation, the
split-K choice, the program's structure, its ordering (the race-checking
simulator), and its result against the oracle.

What the share computes (virtual rank 0 of a one-way ring):
  AllGather->GEMM:  y_0 = act(Xfull . W_0^T), Xfull the N shards in rank order
                    (the oracle's AllGather->GEMM, rank 0's block).
  GEMM->ReduceScatter: step s adds P_s = H_0[b_s rows] . W_0^T, b_s =
                    (N - 1 - s) mod N, to the neighbour's bucket peer[s - 1]
                    (none at s = 0); steps s < N - 1 send the sum (sent[s]),
                    the last one is rank 0's output.  P_s is the oracle's
                    GEMM of one rank (its AllGather->GEMM with N = 1).
Integer inputs: exact in fp32 in any order, so the simulated program's
fp32/bf16 stores equal the oracle's (rounded) values bit for bit.
"""
import numpy as np
import pytest

import oracle
from collective_matmul_decomposition_amd import _native as nat
from collective_matmul_decomposition_amd import inputs as gen

from ring_sim import Sim, buffer_sizes, check_program_bounds


def share_plan(op, N, m, k, n, **kw):
    return nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, share=1, **kw)


def test_share_validation():
    ok = dict(op="ag", n_ranks=4, m=64, k=512, n=256, share=1)
    for kw, want in [(dict(dir="bi"), nat.CM_ERR_UNSUPPORTED), (dict(chunks=2), nat.CM_ERR_UNSUPPORTED),
                     (dict(op="rs", hop="add"), nat.CM_ERR_UNSUPPORTED), (dict(op="rs_pipe"), nat.CM_ERR_UNSUPPORTED),
                     (dict(op="rs", bucket="bf16"), nat.CM_ERR_UNSUPPORTED),
                     (dict(sched="naive"), nat.CM_ERR_UNSUPPORTED), (dict(split_k=3), nat.CM_ERR_SHAPE),
                     (dict(split_k=17), nat.CM_ERR_INVALID_ARG), (dict(share=2), nat.CM_ERR_INVALID_ARG),
                     (dict(share=0, split_k=2), nat.CM_ERR_INVALID_ARG), (dict(dir="direct"), nat.CM_ERR_UNSUPPORTED)]:
        st, _ = nat.cm_ring_plan_status(nat.make_desc(**dict(ok, **kw)))
        assert st == want, kw
    assert nat.cm_ring_plan_status(nat.make_desc(**dict(ok, split_k=4)))[0] == nat.CM_OK


def test_share_split_choice():
    # GPT-3 MLP steps of one rank: fc1 [256 x 12288] . [12288 x 6144] has 32
    # tiles of 256x192 -> 8 slices of 24 slabs fill 256 compute units; fc2
    # [256 x 6144] . [6144 x 12288] has 64 -> 4 slices.
    p = share_plan("ag", 8, 256, 12288, 6144)
    assert (p.split, p.tile_m, p.tile_n) == (8, 256, 192)
    p = share_plan("rs", 8, 256, 6144, 12288)
    assert (p.split, p.tile_m, p.tile_n) == (4, 256, 192)
    # tiny shapes are not split; every slice keeps at least 8 slabs
    assert share_plan("ag", 4, 64, 256, 256).split == 1
    for op, k, n in (("ag", 4096, 1792), ("rs", 1792, 4096), ("ag", 1024, 512)):
        p = share_plan(op, 8, 256, k, n)
        assert (k // 64) % p.split == 0 and (k // 64) // p.split >= 8 or p.split == 1
    assert share_plan("ag", 8, 256, 12288, 6144, split_k=3).split == 3


@pytest.mark.parametrize("op", ["ag", "rs"])
@pytest.mark.parametrize("N,split", [(1, 1), (2, 2), (4, 3), (5, 1)])
def test_share_program_structure(op, N, split):
    m, k, n = 16, 64 * 6, 128
    p = share_plan(op, N, m, k, n, split_k=split, out_dtype="f32", n_comm=2)
    ops, jobs = nat.cm_plan_program(p)
    gemms = [o for o in ops if o.kind == nat.CM_OPK_GEMM]
    reds = [o for o in ops if o.kind == nat.CM_OPK_REDUCE]
    copies = [o for o in ops if o.kind == nat.CM_OPK_COPY]
    assert len(gemms) == N and all(o.n_jobs == split and o.depth == k // split for o in gemms)
    assert len(reds) == N and all(o.n_jobs == 1 and o.depth == split and o.stream == 0 for o in reds)
    assert len(copies) == N - 1
    hop = m * k * 2 if op == "ag" else m * n * 4
    assert all(c.bytes == hop and c.stream == 1 for c in copies)
    # every job of a step GEMM is rank 0's, slice i of K
    for o in gemms:
        js = jobs[o.first_job:o.first_job + o.n_jobs]
        assert [j.index for j in js] == list(range(split)) and all(j.rank == 0 for j in js)
    check_program_bounds(p)


def _share_data(op, N, m, k, n, dist, seed=1):
    if op == "ag":
        x, w = gen.ag_inputs(N, m, k, n, dist, seed)
        return x, w, None
    h, w = gen.rs_inputs(N, m, k, n, dist, seed)
    return h, w, gen.peer_buckets(N, m, n, dist, seed)


def share_expected(op, a, w, peer, act="none"):
    """What one rank's share must produce, from the oracle: AG -> y_0 [N*m, n];
    RS -> (sent [N-1, m, n], out_0 [m, n]), with the magnitudes for the bound."""
    if op == "ag":
        y, mag = oracle.ag_gemm(a, w, with_mag=True)
        y0, m0 = y[0], mag[0]
        if act == "gelu":
            return oracle.gelu(y0), m0
        return y0, m0
    N, T, k = a.shape
    m = T // N
    sums, mags = [], []
    for s in range(N):
        b = (N - 1 - s) % N
        P, Pm = oracle.ag_gemm(a[0, b * m:(b + 1) * m][None], w[:1], with_mag=True)  # one rank's GEMM
        val, mg = P[0], Pm[0]
        if s >= 1:
            val = val + peer[s - 1].astype(np.float64)
            mg = mg + np.abs(peer[s - 1].astype(np.float64))
        sums.append(val)
        mags.append(mg)
    return (np.stack(sums[:-1]) if N > 1 else np.zeros((0, m, w.shape[1])), sums[-1]), (mags[:-1], mags[-1])


def _run_sim(op, N, m, k, n, dist, split, out_dtype, act="none"):
    p = share_plan(op, N, m, k, n, split_k=split, out_dtype=out_dtype, n_comm=2, act=act)
    a, w, peer = _share_data(op, N, m, k, n, dist)
    sizes = buffer_sizes(p)
    ws = np.zeros(p.ws_bytes, np.uint8)
    if op == "rs" and N > 1:
        ws[:peer.nbytes] = peer.view(np.uint8).reshape(-1)
    data = {nat.CM_BUF_X: a if op == "ag" else a[:1], nat.CM_BUF_W: w[:1], nat.CM_BUF_WS: ws}
    sim = Sim(p, sizes, data).run()
    return p, sim, (a, w, peer)


def _out(sim, b, shape, out_dtype):
    raw = sim.buf[b]
    if out_dtype == "f32":
        return raw.view(np.float32).reshape(shape).astype(np.float64)
    return gen.bf16_bits_to_f32(raw.view(np.uint16).reshape(shape)).astype(np.float64)


@pytest.mark.parametrize("op", ["ag", "rs"])
@pytest.mark.parametrize("N,m,k,n,split", [(1, 8, 128, 64, 2), (2, 5, 256, 128, 4), (4, 8, 192, 64, 3), (3, 16, 512, 192, 0)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_share_sim_equals_oracle_int(op, N, m, k, n, split, out_dtype):
    p, sim, (a, w, peer) = _run_sim(op, N, m, k, n, "int", split, out_dtype)
    if op == "ag":
        want, _ = share_expected(op, a, w, peer)
        got = _out(sim, nat.CM_BUF_Y, (N * m, n), out_dtype)
        assert np.array_equal(got, want if out_dtype == "f32" else gen.bf16_bits_to_f32(oracle.round_bf16(want)))
    else:
        (sent, out0), _ = share_expected(op, a, w, peer)
        got = _out(sim, nat.CM_BUF_Y, (m, n), out_dtype)
        assert np.array_equal(got, out0 if out_dtype == "f32" else gen.bf16_bits_to_f32(oracle.round_bf16(out0)))
        if N > 1:
            L = (N - 1) * m * n * 4 + 2 * m * n * 4  # the sent buckets follow the peer buckets and the slots
            got_sent = sim.buf[nat.CM_BUF_WS][L:L + (N - 1) * m * n * 4].view(np.float32).reshape(N - 1, m, n)
            assert np.array_equal(got_sent.astype(np.float64), sent)


def test_share_sim_gelu_normal():
    N, m, k, n = 3, 8, 256, 64
    p, sim, (a, w, peer) = _run_sim("ag", N, m, k, n, "normal", 2, "f32", act="gelu")
    want, _ = share_expected("ag", a, w, peer, act="gelu")
    got = _out(sim, nat.CM_BUF_Y, (N * m, n), "f32")
    assert np.allclose(got, want, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("op", ["ag", "rs"])
def test_share_dropped_wait_is_caught(op):
    """Negative control: removing any one in-schedule wait of the share
    program (hop after the slot's last reader, step after its arrival) races."""
    from test_plan import _drop_op
    from ring_sim import Race
    N, m, k, n = 4, 8, 256, 64
    p = share_plan(op, N, m, k, n, split_k=2, out_dtype="f32", n_comm=2)
    a, w, peer = _share_data(op, N, m, k, n, "int")
    ws = np.zeros(p.ws_bytes, np.uint8)
    if op == "rs":
        ws[:peer.nbytes] = peer.view(np.uint8).reshape(-1)
    data = {nat.CM_BUF_X: a if op == "ag" else a[:1], nat.CM_BUF_W: w[:1], nat.CM_BUF_WS: ws}
    sizes = buffer_sizes(p)
    base = Sim(p, sizes, data)
    waits = [i for i, o in enumerate(base.ops) if o.kind == nat.CM_OPK_WAIT and o.step >= 0]
    assert len(waits) == (N - 1) + (N - 3)  # each step after its arrival; hops s >= 2 after the slot's last reader
    for i in waits:
        with pytest.raises(Race):
            _drop_op(Sim(p, sizes, data), i).run()
