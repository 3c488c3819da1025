"""Compile the CPU oracle (oracle.c) into oracle/_liboracle.so with gcc.

Test infrastructure: the library built here is loaded only by the test suite,
the smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "_liboracle.so")


def build(verbose: bool = False, lib: str = LIB, cc: str = "gcc", flags=()) -> str:
    """Compile oracle.c into `lib` (another compiler and extra flags serve a
    sanitizer build into another path)."""
    src = os.path.join(HERE, "oracle.c")
    tmp = lib + ".tmp"
    cmd = [cc, "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-fopenmp"] + list(flags) + ["-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
