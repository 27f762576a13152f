"""Compile the FP64 softmax oracle (plain C, gcc, OpenMP) into oracle/liboracle_softmax.so.

Test infrastructure: the oracle is a checker, built next to the GPU library so the
tests can load it. It is never linked into the product.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_softmax.c")
LIB = os.path.join(HERE, "liboracle_softmax.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
        "-fPIC", "-shared", SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
