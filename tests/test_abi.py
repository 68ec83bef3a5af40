"""The C ABI on the CPU: every declared symbol is exported, and invalid
requests and calls fail with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

from collective_matmul_decomposition_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "collmm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = nat.lib()
    names = declared_functions()
    assert len(names) >= 11, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(nat.EXPORTS)


def test_struct_sizes_match_the_header():
    # compile a tiny C program against the header and compare sizeof
    import subprocess
    import tempfile
    src = r'''
#include <stdio.h>
#include "collmm.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(cm_plan_desc), sizeof(cm_plan), sizeof(cm_op_rec),
         sizeof(cm_job_rec), sizeof(cm_span), sizeof(cm_layer_desc), sizeof(cm_layer_plan), sizeof(cm_bwd_desc),
         sizeof(cm_bwd_plan));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        sizes = [int(v) for v in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert sizes == [ctypes.sizeof(nat.cm_plan_desc), ctypes.sizeof(nat.cm_plan), ctypes.sizeof(nat.cm_op_rec),
                     ctypes.sizeof(nat.cm_job_rec), ctypes.sizeof(nat.cm_span), ctypes.sizeof(nat.cm_layer_desc),
                     ctypes.sizeof(nat.cm_layer_plan), ctypes.sizeof(nat.cm_bwd_desc), ctypes.sizeof(nat.cm_bwd_plan)]


def status_of(**kw):
    base = dict(op="ag", n_ranks=4, m=64, k=256, n=256)
    base.update(kw)
    st, _ = nat.cm_ring_plan_status(nat.make_desc(**base))
    return st


@pytest.mark.parametrize("kw,expect", [
    (dict(), nat.CM_OK),
    (dict(n_ranks=0), nat.CM_ERR_INVALID_ARG),
    (dict(n_ranks=65), nat.CM_ERR_INVALID_ARG),
    (dict(op=7), nat.CM_ERR_INVALID_ARG),
    (dict(dir=5), nat.CM_ERR_INVALID_ARG),
    (dict(sched=3), nat.CM_ERR_INVALID_ARG),
    (dict(n_comm=0), nat.CM_ERR_INVALID_ARG),
    (dict(n_comm=33), nat.CM_ERR_INVALID_ARG),
    (dict(k=100), nat.CM_ERR_SHAPE),
    (dict(n=96), nat.CM_ERR_SHAPE),
    (dict(m=0), nat.CM_ERR_SHAPE),
    (dict(chunks=3), nat.CM_ERR_SHAPE),              # 3 does not divide m = 64
    (dict(op="rs", chunks=3), nat.CM_ERR_SHAPE),     # 256 / 3
    (dict(op="rs", chunks=8), nat.CM_ERR_SHAPE),     # 256 / 8 = 32 columns, not a multiple of 64
    (dict(chunks=17), nat.CM_ERR_SHAPE),
    (dict(out_dtype=5), nat.CM_ERR_UNSUPPORTED),
    (dict(tile=(96, 96)), nat.CM_ERR_UNSUPPORTED),
    (dict(exec_mode=4), nat.CM_ERR_INVALID_ARG),
    (dict(copy_engine=3), nat.CM_ERR_INVALID_ARG),
])
def test_plan_validation(kw, expect):
    assert status_of(**kw) == expect
    if expect != nat.CM_OK:
        assert nat.last_error() != ""


def test_status_strings():
    lib = nat.lib()
    for st in range(8):
        assert lib.cm_status_string(st).decode().startswith("CM_")


def _call(fn, plan, ptrs=(16, 32, 48, 64), ws_bytes=None, n_comm=None, comm=None):
    n_comm = plan.desc.n_comm if n_comm is None else n_comm
    comm = comm if comm is not None else [1000 + 16 * i for i in range(n_comm)]
    arr = (ctypes.c_void_p * max(1, len(comm)))(*comm)
    ws_bytes = plan.ws_bytes if ws_bytes is None else ws_bytes
    return fn(ctypes.byref(plan), ptrs[0], ptrs[1], ptrs[2], ptrs[3], ws_bytes, 4096, arr, n_comm, None)


def test_call_validation_happens_before_any_hip_call():
    lib = nat.lib()
    plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=64, k=256, n=256, n_comm=2)
    rs_plan = nat.cm_ring_plan(op="rs", n_ranks=4, m=64, k=256, n=256, n_comm=2)
    ag, rs = lib.cm_ag_gemm, lib.cm_gemm_rs
    assert _call(ag, rs_plan) == nat.CM_ERR_INVALID_ARG           # wrong op for the entry point
    assert _call(rs, plan) == nat.CM_ERR_INVALID_ARG
    assert _call(ag, plan, ptrs=(0, 32, 48, 64)) == nat.CM_ERR_INVALID_ARG
    assert _call(ag, plan, ptrs=(16, 32, 48, 0)) == nat.CM_ERR_INVALID_ARG
    assert _call(ag, plan, ptrs=(17, 32, 48, 64)) == nat.CM_ERR_ALIGN
    assert _call(ag, plan, ws_bytes=plan.ws_bytes - 1) == nat.CM_ERR_WORKSPACE
    assert _call(ag, plan, n_comm=1, comm=[1000]) == nat.CM_ERR_INVALID_ARG
    assert _call(ag, plan, comm=[1000, 1000]) == nat.CM_ERR_INVALID_ARG   # the same stream twice
    assert _call(ag, plan, comm=[1000, 0]) == nat.CM_ERR_INVALID_ARG      # a null comm stream
    assert _call(ag, plan, comm=[1000, 4096]) == nat.CM_ERR_INVALID_ARG   # comm == compute
    bad = nat.cm_plan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    bad.n_steps += 1                                                    # a plan cm_ring_plan did not make
    assert _call(ag, bad) != nat.CM_OK
    bad.n_steps -= 1
    bad.ws_bytes += 16
    assert _call(ag, bad) == nat.CM_ERR_INVALID_ARG


def test_program_query_capacity():
    lib = nat.lib()
    plan = nat.cm_ring_plan(op="rs", n_ranks=4, m=64, k=256, n=256, chunks=2, n_comm=2)
    n_ops, n_jobs = ctypes.c_int(), ctypes.c_int()
    assert lib.cm_plan_program(ctypes.byref(plan), None, 0, ctypes.byref(n_ops), None, 0, ctypes.byref(n_jobs)) == 0
    assert n_ops.value == plan.n_ops and n_jobs.value == plan.n_jobs
    ops = (nat.cm_op_rec * 1)()
    jobs = (nat.cm_job_rec * 1)()
    assert lib.cm_plan_program(ctypes.byref(plan), ops, 1, ctypes.byref(n_ops), jobs, 1,
                               ctypes.byref(n_jobs)) == nat.CM_ERR_CAPACITY


def test_workspace_size_and_version():
    plan = nat.cm_ring_plan(op="ag", n_ranks=4, m=64, k=256, n=256, dir="bi", n_comm=2)
    assert nat.cm_workspace_size(plan) == plan.ws_bytes == 2 * 2 * 4 * 64 * 256 * 2
    assert re.match(r"^\d+\.\d+\.\d+$", nat.version())


def test_trace_argument_checks():
    lib = nat.lib()
    h = ctypes.c_void_p()
    assert lib.cm_trace_create(0, ctypes.byref(h)) == nat.CM_ERR_INVALID_ARG
    assert lib.cm_trace_destroy(None) == nat.CM_OK


class _FakeTensor:
    """Stands in for a torch tensor on the GPU (the checks run before any call)."""

    def __init__(self, numel, dtype="bfloat16", contiguous=True, device="cuda"):
        self._n, self.dtype, self._c = numel, "torch." + dtype, contiguous
        self.device = type("D", (), {"type": device})()

    def numel(self):
        return self._n

    def element_size(self):
        return {"bfloat16": 2, "float16": 2, "float32": 4, "uint8": 1}[self.dtype.split(".")[-1]]

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        raise AssertionError("the library must not be called")


@pytest.mark.parametrize("bad", ["x_small", "w_dtype", "y_small", "y_dtype", "ws_small", "noncontig", "cpu"])
def test_binding_rejects_bad_tensors_before_calling(bad):
    """Tensor arguments are checked against the plan's layout on the host, so a
    buffer that is too small becomes a Python error, not out-of-bounds writes."""
    N, m, k, n = 4, 16, 64, 128
    plan = nat.cm_ring_plan(op="ag", n_ranks=N, m=m, k=k, n=n, out_dtype="f32")
    args = dict(x=_FakeTensor(N * m * k), w=_FakeTensor(N * n * k), y=_FakeTensor(N * N * m * n, "float32"),
                ws=_FakeTensor(max(1, plan.ws_bytes), "uint8"))
    if bad == "x_small":
        args["x"] = _FakeTensor(N * m * k - 1)
    elif bad == "w_dtype":
        args["w"] = _FakeTensor(N * n * k, "float16")
    elif bad == "y_small":
        args["y"] = _FakeTensor(N * N * m * n - 8, "float32")
    elif bad == "y_dtype":
        args["y"] = _FakeTensor(N * N * m * n, "bfloat16")
    elif bad == "ws_small":
        args["ws"] = _FakeTensor(plan.ws_bytes - 1, "uint8")
    elif bad == "noncontig":
        args["x"] = _FakeTensor(N * m * k, contiguous=False)
    elif bad == "cpu":
        args["w"] = _FakeTensor(N * n * k, device="cpu")
    with pytest.raises(ValueError):
        nat.cm_ag_gemm(plan, args["x"], args["w"], args["y"], args["ws"], None, [])
