"""Inline-asm vector loads in the GEMM kernels, checked in the gfx950
assembly that the build flags produce (CPU only: hipcc cross-compiles).

The kernels issue every load through compiler builtins, whose waits the
compiler inserts itself.  A load written as inline asm with an explicit
`s_waitcnt vmcnt` is only correct while the compiler leaves its destination
registers alone until the wait; `asm_flow` checks that by dataflow, and the
build requires that no such load exists at all.
"""
import os
import shutil
import subprocess

import pytest

from collective_matmul_decomposition_amd import asm_check as asm_flow
from collective_matmul_decomposition_amd import build as B


@pytest.fixture(scope="module")
def kernels_asm(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "kernels.s")
    cmd = [B.HIPCC, *B.COMMON, *B.DEVICE, "--cuda-device-only", "-S", os.path.join(B.CSRC, "kernels.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def test_build_check_fails_on_a_planted_asm_load(tmp_path):
    """The same check runs in build(): a source mutant that issues a load
    through inline asm makes it fail."""
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    src = open(os.path.join(B.CSRC, "kernels.hip")).read()
    anchor = "  f32x16 acc[TM][TN];\n"
    assert anchor in src
    planted = ("  { i32x4 v; asm volatile(\"global_load_dwordx4 %0, %1, off\\n s_waitcnt vmcnt(0)\" : \"=v\"(v) : \"v\"(Abase) : \"memory\");\n"
               "    asm volatile(\"\" :: \"v\"(v)); }\n") + anchor
    mutant = tmp_path / "kernels.hip"
    mutant.write_text(src.replace(anchor, planted, 1))
    with pytest.raises(RuntimeError, match="GEMM"):
        B.check_loader_asm(str(mutant), str(tmp_path / "kernels.s"))


def test_kernels_have_no_asm_loads(kernels_asm):
    checked = 0
    for name, lines in asm_flow.functions(kernels_asm).items():
        n, bad = asm_flow.analyse(lines)
        if n == 0:
            continue
        checked += 1
        assert not bad, "%s: %d instructions touch in-flight load registers, e.g. %s" % (name, len(bad), bad[:5])
    assert checked == 0


# A planted mistake on hand-written assembly: the analysis must flag a copy of
# a register whose load is in flight, a spill of it, and an address computed
# into it, and accept the intended store-after-wait pattern.
GOOD = """_Zgood:
\t;;#ASMSTART
\tglobal_load_dwordx4 v[2:5], v0, s[4:5]
\t;;#ASMEND
\t;;#ASMSTART
\tglobal_load_dwordx4 v[6:9], v1, s[4:5]
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt vmcnt(1)
\t;;#ASMEND
\tds_write_b128 v10, v[2:5]
\t;;#ASMSTART
\ts_waitcnt vmcnt(0)
\t;;#ASMEND
\tv_mov_b32_e32 v2, 0
\ts_endpgm
.Lfunc_end0:
"""


def _variant(extra_after_loads):
    return GOOD.replace("\t;;#ASMSTART\n\ts_waitcnt vmcnt(1)", extra_after_loads + "\t;;#ASMSTART\n\ts_waitcnt vmcnt(1)")


@pytest.mark.parametrize("planted", ["\tv_mov_b32_e32 v20, v7\n", "\tv_accvgpr_write_b32 a3, v4\n",
                                     "\tscratch_store_dword off, v11, s33\n", "\tv_add_u32_e32 v8, 16, v0\n"])
def test_planted_violation_is_flagged(planted):
    (lines,) = asm_flow.functions(GOOD).values()
    assert asm_flow.analyse(lines) == (2, [])
    (lines,) = asm_flow.functions(_variant(planted)).values()
    n, bad = asm_flow.analyse(lines)
    assert n == 2 and bad == [planted.strip()]


def test_branch_paths_merge():
    """A register loaded on one path of a branch is in flight after the merge."""
    asm = """_Zbr:
\ts_cbranch_scc0 .LBB0_2
\t;;#ASMSTART
\tglobal_load_dwordx4 v[2:5], v0, s[4:5]
\t;;#ASMEND
.LBB0_2:
\tv_mov_b32_e32 v6, v3
\ts_endpgm
.Lfunc_end0:
"""
    (lines,) = asm_flow.functions(asm).values()
    assert asm_flow.analyse(lines)[1] == ["v_mov_b32_e32 v6, v3"]
