"""Builds the CPU oracle (test infrastructure only) into oracle/liblsa_ref.so with gcc.

Plain C, IEEE fp64: no fast-math and no floating-point contraction, so every sum is the
index-order sum the source spells out.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lsa_ref.c")
LIB = os.path.join(HERE, "liblsa_ref.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", LIB, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
