"""Device buffers and streams for a plan (torch is used only as an allocator).

Sizes follow the layouts of include/collmm.h:
    AllGather->GEMM   x [N, m, k] bf16, w [N, n, k] bf16, y [N, N*m, n]
    GEMM->ReduceScatter x [N, N*m, k] bf16, w [N, n, k] bf16, y [N, m, n]
and for one rank's share (plan.desc.share = 1) rank 0's blocks:
    AllGather->GEMM   x [N, m, k] (all shards), w [1, n, k], y [1, N*m, n]
    GEMM->ReduceScatter x [1, N*m, k], w [1, n, k], y [1, m, n]
plus the plan's workspace (plan.ws_bytes, at least one byte so it has an
address).
"""
from . import _native as nat


def shapes(plan):
    d = plan.desc
    N, m, k, n = d.n_ranks, d.m, d.k, d.n
    T = N * m
    R = 1 if d.share else N  # ranks whose weights and outputs the call touches
    if d.op == nat.CM_OP_AG_GEMM:
        return {"x": (N, m, k), "w": (R, n, k), "y": (R, T, n)}
    return {"x": (R, T, k), "w": (R, n, k), "y": (R, m, n)}


def alloc_outputs(plan, device="cuda"):
    """(y, ws) torch tensors for a plan."""
    import torch
    ydt = torch.float32 if plan.desc.out_dtype == nat.CM_F32 else torch.bfloat16
    y = torch.empty(shapes(plan)["y"], dtype=ydt, device=device)
    ws = torch.empty(max(1, plan.ws_bytes), dtype=torch.uint8, device=device)
    return y, ws


def check_inputs(plan, x, w, y, ws):
    """Host-side check that the tensors match the plan's layout (before any launch)."""
    import torch
    sh = shapes(plan)
    if tuple(x.shape) != sh["x"] or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 tensor of shape %s, got %s %s" % (sh["x"], tuple(x.shape), x.dtype))
    if tuple(w.shape) != sh["w"] or w.dtype != torch.bfloat16 or not w.is_contiguous():
        raise ValueError("w must be a contiguous bf16 tensor of shape %s, got %s %s" % (sh["w"], tuple(w.shape), w.dtype))
    ydt = torch.float32 if plan.desc.out_dtype == nat.CM_F32 else torch.bfloat16
    if tuple(y.shape) != sh["y"] or y.dtype != ydt or not y.is_contiguous():
        raise ValueError("y must be a contiguous %s tensor of shape %s" % (ydt, sh["y"]))
    if ws.numel() * ws.element_size() < plan.ws_bytes or not ws.is_contiguous():
        raise ValueError("workspace smaller than the plan's %d bytes" % plan.ws_bytes)
    for t in (x, w, y, ws):
        if t.device.type != "cuda":
            raise ValueError("all buffers must be on the GPU")


def comm_streams(n_comm, device="cuda"):
    """n_comm new streams at the default priority."""
    import torch
    return [torch.cuda.Stream(device=device) for _ in range(n_comm)]


def run(plan, x, w, y, ws, compute=None, comm=None, trace=None):
    """Check the buffers on the host, then call cm_ag_gemm / cm_gemm_rs."""
    import torch
    check_inputs(plan, x, w, y, ws)
    if compute is None:
        compute = torch.cuda.current_stream()
    if comm is None:
        comm = comm_streams(plan.desc.n_comm)
    fn = nat.cm_ag_gemm if plan.desc.op == nat.CM_OP_AG_GEMM else nat.cm_gemm_rs
    fn(plan, x, w, y, ws, compute, comm, trace)
    return comm
