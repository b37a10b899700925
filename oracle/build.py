"""Build the CPU oracle (test infrastructure only) into oracle/libcsa2_oracle.so.

Plain gcc, -O2, no fast-math and no FP contraction, so every float expression
in csa2_oracle.c is the IEEE operation it reads as.  OpenMP only splits
independent queries across threads; per-query arithmetic is unchanged.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcsa2_oracle.so")
FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-fopenmp", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose=False):
    src = os.path.join(HERE, "csa2_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", *FLAGS, src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
