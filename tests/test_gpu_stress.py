"""GPU race stress of the programs' ordering (the eager executor's stress
mode): seeded sleeps before operations shift the streams against each other,
and every workspace region is filled with 0xFF (NaN) right before it is
overwritten, so a reader that is not ordered before the next writer reads
poison, and a consumer not ordered after its producer reads stale data or
poison.  With the ordering right the outputs equal those of the run without
stress bit for bit (the Megatron page, section 5: a bucket may be overwritten
only after every later reader is done, and read only after its producer).
Each case stops at its first mismatch.
"""
import sys

import numpy as np
import pytest

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


CASES = [
    # op, N, m, k, n, dir, chunks, n_comm, hop, sched
    ("ag", 4, 64, 256, 256, "uni", 1, 1, "copy", "decomposed"),       # the tiny configuration
    ("rs", 4, 64, 256, 256, "uni", 2, 1, "copy", "decomposed"),
    ("ag", 8, 32, 512, 256, "bi", 2, 2, "copy", "decomposed"),
    ("rs", 8, 32, 256, 512, "bi", 1, 2, "add", "decomposed"),
    ("rs", 8, 32, 256, 512, "uni", 1, 1, "add", "decomposed"),
    ("rs", 5, 40, 192, 256, "uni", 2, 3, "copy", "decomposed"),
    ("ag", 5, 40, 192, 256, "direct", 1, 2, "copy", "decomposed"),
    ("rs", 5, 40, 192, 256, "direct", 2, 2, "copy", "decomposed"),
    ("rs_pipe", 4, 64, 256, 512, "uni", 4, 1, "add", "decomposed"),
    ("rs_pipe", 4, 64, 256, 512, "uni", 2, 2, "copy", "decomposed"),
    ("ag", 4, 128, 512, 512, "uni", 1, 1, "copy", "naive"),
    ("rs", 4, 128, 512, 512, "uni", 1, 1, "copy", "naive"),
    # the small-chunk regime (d = 2048, ffn 8192, 1024 tokens) at N = 4
    ("ag", 4, 256, 2048, 2048, "uni", 4, 1, "copy", "decomposed"),
    ("rs", 4, 256, 2048, 2048, "uni", 4, 1, "copy", "decomposed"),
]


def run(op, N, m, k, n, dir, chunks, n_comm, hop, sched, a_t, w_t, stress, share=0):
    plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, n_comm=n_comm,
                            hop=hop if op != "ag" else "copy", sched=sched, out_dtype="f32", exec_mode="eager",
                            stress=stress, share=share)
    y, ws = buffers.alloc_outputs(plan)
    y.fill_(float("nan"))
    if share and op == "rs":
        # the arriving buckets (the caller's, at the start of the workspace): small integers
        peer = torch.randint(-40, 41, ((N - 1) * m * n,), device="cuda").float()
        ws[:peer.numel() * 4].view(torch.float32).copy_(peer)
    buffers.run(plan, a_t, w_t, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_stress_keeps_results(case):
    op, N, m, k, n, dir, chunks, n_comm, hop, sched = case
    mk = gen.ag_inputs if op == "ag" else gen.rs_inputs
    a, w = mk(N, m, k, n, "int", 3)
    a_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    say("stress", case, "reference")
    ref = run(*case, a_t, w_t, 0)
    assert not torch.isnan(ref).any()
    for seed in (1, 2, 3):
        say("stress", case, "seed", seed)
        got = run(*case, a_t, w_t, seed)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), "seed %d changed the results" % seed


@pytest.mark.parametrize("op", ["ag", "rs"])
def test_stress_one_rank_share(op):
    N, m, k, n = 4, 64, 1024, 256
    if op == "ag":
        a, w = gen.ag_inputs(N, m, k, n, "int", 5)
        w = w[:1]
    else:
        a, w = gen.rs_inputs(N, m, k, n, "int", 5)
        a, w = a[:1], w[:1]
    a_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    torch.manual_seed(0)
    ref = run(op, N, m, k, n, "uni", 1, 1, "copy", "decomposed", a_t, w_t, 0, share=1)
    for seed in (1, 2):
        torch.manual_seed(0)  # the same arriving buckets
        say("stress share", op, "seed", seed)
        got = run(op, N, m, k, n, "uni", 1, 1, "copy", "decomposed", a_t, w_t, seed, share=1)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), "seed %d changed the results" % seed
