"""The GEMM loader's asynchronously written registers, checked in the gfx950
assembly that the build flags produce (CPU only: hipcc cross-compiles).

The loader waves of the register-staged GEMM instantiations issue their
global loads as inline asm and store each register set to LDS after an
explicit partial `s_waitcnt vmcnt`.  This is only correct while the compiler
leaves those registers alone until the wait; `asm_flow` proves that for the
code as built, and fails if a compiler or code change copies, spills or
reuses one of them while its load may be in flight.  The wait counts
themselves are checked against the issue order in `test_wait_counts`.
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


def test_build_check_fails_on_a_planted_read(tmp_path):
    """The same check runs in build(): a source mutant whose loader reads a
    register of a load that may still be in flight makes it fail."""
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    src = open(os.path.join(B.CSRC, "kernels.hip")).read()
    anchor = "    for (int j = 0; j < RS; ++j) gload(j, j);\n"
    assert anchor in src
    planted = anchor + ("    { int sink; asm volatile(\"v_mov_b32 %0, %1\" : \"=v\"(sink) : \"v\"(ra[0][0][0]));\n"
                        "      asm volatile(\"\" :: \"v\"(sink)); }\n")
    mutant = tmp_path / "kernels.hip"
    mutant.write_text(src.replace(anchor, planted))
    with pytest.raises(RuntimeError, match="in-flight"):
        B.check_loader_asm(str(mutant), str(tmp_path / "kernels.s"))


def test_loader_registers_untouched_until_waited(kernels_asm):
    checked = 0
    for name, lines in asm_flow.functions(kernels_asm).items():
        n, bad = asm_flow.analyse(lines)
        if n == 0:
            continue
        checked += 1
        assert not bad, "%s: %d instructions touch in-flight load registers, e.g. %s" % (name, len(bad), bad[:5])
    # the register-staged 256x192 tile, with and without epilogue addends
    assert checked == 2


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


def test_wait_counts():
    """The loader stores slab j after a wait that leaves outstanding exactly
    the loads issued after slab j's: those of slabs j+1 .. j+RS-1 (the ones
    that exist).  Simulated over the issue order (RS register sets, SB LDS
    slabs, LA + LB loads per slab) for short and long K loops."""
    for RS in (2, 3, 4):
        for SB in (2, 3):
            for KT in range(1, 12):
                L = 14
                issued = []  # slab of each load, in issue order

                def gload(s):
                    if s < KT:
                        issued.extend([s] * L)

                def lstore(s):
                    if s >= KT:
                        return
                    younger = sum(L for q in range(1, RS) if s + q < KT)  # the kernel's count
                    last = max(i for i, x in enumerate(issued) if x == s)
                    assert len(issued) - 1 - last == younger, (RS, SB, KT, s)
                    # slab s's register set (s mod RS) has not yet been reloaded
                    assert s + RS not in issued

                for j in range(RS):
                    gload(j)
                for j in range(SB - 1):
                    lstore(j)
                    gload(j + RS)
                for kt in range(KT):
                    lstore(kt + SB - 1)
                    gload(kt + SB - 1 + RS)
