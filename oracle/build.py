"""Compile the CPU oracle (pa_oracle.c) into oracle/libpa_oracle.so with gcc.

Test infrastructure: the library built here is loaded only by the test suite,
the smoke check and the CPU-baseline leg of the benchmark.

Flags: -O2 with -ffp-contract=off and no fast-math, so that every double
operation is an IEEE-754 round-to-nearest operation in source order; OpenMP
parallelises over independent output rows only, which does not change any
row's arithmetic.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "libpa_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
