"""Build the CPU oracle's shared library (test infrastructure only).

gcc, -O2, no fused multiply-add contraction, no fast-math, OpenMP across
independent output rows.  Run as ``python -m oracle.build`` or call
``build()``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "psi_oracle.c")
LIB = os.path.join(HERE, "libpsi_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
