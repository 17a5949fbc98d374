"""Builds the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

The oracle is test infrastructure: only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.  -ffp-contract=off keeps every
multiply and add a separate IEEE operation, as the C source reads.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
