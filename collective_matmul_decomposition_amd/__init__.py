"""libcollmm: decomposed tensor-parallel AllGather->GEMM and GEMM->ReduceScatter
for MI355X (gfx950).

The compute path is the C-ABI library libcollmm.so (HIP kernels, SDMA ring
hops, event ordering); this package is its ctypes binding plus the seeded
input generators.  Build the library with
`python -m collective_matmul_decomposition_amd.build`.
"""
from ._native import (  # noqa: F401
    CMError, Trace, cm_ag_gemm, cm_gemm_rs, cm_plan, cm_plan_desc, cm_plan_program, cm_ring_plan,
    cm_workspace_size, last_error, lib, make_desc, version,
)
