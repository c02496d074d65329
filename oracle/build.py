"""Build the CPU oracle (test infrastructure) into ``oracle/liboracle.so`` with gcc.

Plain C, binary64, no fast-math and no FMA contraction, so every product and
comparison in the oracle is the IEEE operation it is written as.  OpenMP is used
only to spread independent rows over host cores.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build for the sanitized CPU test run:
# clang (the ROCm toolchain's, whose sanitizer runtime the HIP library's host code
# uses too), single-threaded (no OpenMP), every UB report fatal
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
CLANG = "/opt/rocm/lib/llvm/bin/clang"


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    cmd = [CLANG, "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra", "-o", SAN_LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
