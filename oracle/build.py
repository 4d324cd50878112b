"""Compile the fp64 CPU oracle into oracle/liboracle.so with gcc.

Test infrastructure only (see oracle.h).  Plain C11, OpenMP over independent
tokens, no fast-math and no FMA contraction, so every sum is the serial fp64
sum written in oracle.c.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile `src` (default oracle.c) into the shared library `lib`."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-I", HERE, src, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
