"""Builds the CPU oracle library (test infrastructure only).

``python -m oracle.build`` or ``build()`` compiles ``conv_oracle.c`` with gcc
into ``liboracle_conv.so`` beside it.  Plain C, -O2, OpenMP, no fast-math:
the oracle's sums must follow IEEE double arithmetic exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv_oracle.c")
LIB = os.path.join(HERE, "liboracle_conv.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
