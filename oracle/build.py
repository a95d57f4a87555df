"""Builds the oracle's shared library (test infrastructure) with gcc.

Portable x86-64 code (no -march=native: the library built here also runs on
other hosts), no fast-math and no FMA contraction, so that the fp64 arithmetic
is exactly what rac_oracle.c spells out.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "rac_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile ``src`` into the shared library ``out`` (atomically replaced)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
