"""GPU: cm_gemm_rs_noalloc (the workspace in the library's static device
array) against cm_gemm_rs with a caller-provided workspace, through the C ABI,
on two calls in a row, the second with a smaller input."""
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


def run_both(N, m, k, n, dist, seed, dir, hop, chunks, out):
    plan = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, out_dtype=out, n_comm=1,
                            hop=hop)
    a, w = gen.rs_inputs(N, m, k, n, dist, seed)
    x_t, w_t = gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda")
    y_ref, ws = buffers.alloc_outputs(plan)
    y_static, _ = buffers.alloc_outputs(plan)
    y_static.fill_(float("nan"))
    comm = buffers.comm_streams(1)
    compute = torch.cuda.current_stream()
    say("noalloc rs N=%d m=%d k=%d n=%d %s dir=%s hop=%s c=%d out=%s ws=%d" % (N, m, k, n, dist, dir, hop,
                                                                             plan.chunks, out, plan.ws_bytes))
    nat.cm_gemm_rs(plan, x_t, w_t, y_ref, ws, compute, comm)
    nat.cm_gemm_rs_noalloc(plan, x_t, w_t, y_static, compute, comm)
    torch.cuda.synchronize()
    return y_ref, y_static


@pytest.mark.parametrize("dir,hop,chunks", [("uni", "copy", 2), ("uni", "add", 1), ("bi", "add", 1),
                                            ("bi", "copy", 2)])
@pytest.mark.parametrize("dist,out", [("int", "f32"), ("normal", "bf16")])
def test_noalloc_equals_workspace_call(dir, hop, chunks, dist, out):
    # first call, then a second, smaller one: the static array keeps the first
    # call's contents, which the second must not depend on
    for (N, m, k, n), seed in (((8, 96, 320, 512), 0), ((4, 40, 192, 256), 1)):
        y_ref, y_static = run_both(N, m, k, n, dist, seed, dir, hop, chunks, out)
        assert torch.equal(y_ref.view(torch.int16) if out == "bf16" else y_ref.view(torch.int32),
                           y_static.view(torch.int16) if out == "bf16" else y_static.view(torch.int32))


def test_noalloc_rejects_plans_beyond_the_static_workspace():
    plan = nat.cm_ring_plan(op="rs", n_ranks=8, m=4096, k=512, n=8192, out_dtype="f32", n_comm=1, chunks=1)
    assert plan.ws_bytes > nat.CM_NOALLOC_WS_BYTES
    st = nat.cm_gemm_rs_noalloc_status(plan)
    assert st == nat.CM_ERR_WORKSPACE
    assert "static" in nat.last_error()
