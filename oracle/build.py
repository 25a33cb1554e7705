"""Build the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is the checker for the HIP library and is
never linked into it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add; no -ffast-math: IEEE semantics.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose=False):
    srcs = [os.path.join(HERE, f) for f in ("qmm_oracle.c", "fp_oracle.c")]
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, *srcs, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
