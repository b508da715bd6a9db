"""Compile the fp64 CPU oracle (test infrastructure) into oracle/libmoe_oracle.so.

Plain C, gcc -O2 -fopenmp, no BLAS and no intrinsics.  Building the checker is
not using it: only tests, the smoke check and the benchmark's CPU-baseline leg
load the library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose=False):
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-shared",
           "-fPIC", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
