"""Builds the oracle's shared library (test infrastructure) with gcc.

Portable x86-64 code (no -march=native: the library built here also runs on
other hosts), no fast-math and no FMA contraction, so that the fp64 arithmetic
is exactly what rac_oracle.c spells out.

With sanitize=True (or ORACLE_SANITIZE=1 in the environment, which the
mutant tests' builds follow too) it is built by the ROCm clang with
AddressSanitizer and UndefinedBehaviorSanitizer instead, for runs of the CPU
tests with that clang's ASan runtime preloaded (see tests/conftest.py).
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "rac_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")


CLANG = "/opt/rocm/llvm/bin/clang"
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g", "-shared-libsan"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB, sanitize=None) -> str:
    """Compile ``src`` into the shared library ``out`` (atomically replaced)."""
    if sanitize is None:
        sanitize = os.environ.get("ORACLE_SANITIZE") == "1"
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    if sanitize:
        cmd = [CLANG, "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"] + \
            SANITIZE_FLAGS + ["-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    if "--sanitize" in sys.argv:
        root = os.path.dirname(_HERE)
        print(build(verbose=True, out=os.path.join(root, "_build", "asan", "liboracle.so"),
                    sanitize=True))
    else:
        print(build(verbose=True))
