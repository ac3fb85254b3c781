"""Builds the CPU oracle (test infrastructure only) into oracle/liblsa_ref.so with gcc.

Plain C, IEEE fp64: no fast-math and no floating-point contraction, so every sum is the
index-order sum the source spells out.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lsa_ref.c")
LIB = os.path.join(HERE, "liblsa_ref.so")


SAN_LIB = os.path.join(HERE, "liblsa_ref_asan.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (CPU only; load it with
# LSA_ORACLE_LIB and gcc's libasan preloaded into the Python process).
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    opt = SAN_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
