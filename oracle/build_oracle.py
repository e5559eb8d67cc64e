"""Compile the plain-C oracle into oracle/liboracle.so (test infrastructure).

No fast-math and no floating-point contraction: every fp32 operation of the
oracle is the one written in oracle.c, and fused multiply-adds happen only
where oracle.c calls fmaf explicitly.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
