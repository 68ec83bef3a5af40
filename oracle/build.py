"""Build the CPU oracle library (test infrastructure only).

Compiles oracle.c with gcc into liboracle.so beside it.  The flags keep the
arithmetic plain: no fast-math, no floating-point contraction, so every
accumulation is the written sequence of fp64 multiply and add.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]


def build(extra_flags=(), out=LIB):
    """Compile the oracle; extra_flags (e.g. -D defines) are appended."""
    cmd = ["gcc", *CFLAGS, *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
