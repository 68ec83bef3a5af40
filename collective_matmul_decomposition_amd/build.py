"""Build libcollmm.so in-tree with hipcc for gfx950.

    python -m collective_matmul_decomposition_amd.build

Compiles the planner (plain C++), the executor and the kernels (HIP) and
links them into collective_matmul_decomposition_amd/libcollmm.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcollmm.so")
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for all device code (no v_pk_*_f32).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = [("plan.cpp", False), ("exec.hip", True), ("kernels.hip", True), ("layer.hip", True), ("backward.hip", True),
           ("noalloc.hip", True)]


def _compile(src, is_hip):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *(DEVICE if is_hip else ["-x", "c++"]), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def check_loader_asm(src=None, out=None, expected_functions=0):
    """Compile the GEMM kernels (src: kernels.hip by default) to gfx950
    assembly with the build flags and check their inline-asm vector loads
    (asm_check): the kernels issue every load through builtins, so none may
    appear (expected_functions = 0); any that does must leave its registers
    alone until a wait drains it.  Raises RuntimeError otherwise."""
    from . import asm_check
    src = src or os.path.join(CSRC, "kernels.hip")
    out = out or os.path.join(OBJDIR, "kernels.s")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [HIPCC, *COMMON, *DEVICE, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("assembly listing failed: %s\n%s" % (" ".join(cmd), r.stderr))
    with open(out) as f:
        return asm_check.check_loader_asm(f.read(), expected_functions)


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        asm = ex.submit(check_loader_asm)
        objs = list(ex.map(lambda s: _compile(*s), SOURCES))
        asm.result()  # raises if the loader's in-flight registers are touched
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", *DEVICE, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
