"""Build the CPU oracle's shared library (test infrastructure only).

Plain single-threaded C, compiled without fast-math and without FMA
contraction so every operation rounds once, in the order the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")


def build(verbose: bool = False, lib: str = LIB, extra_flags=None) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
        "-Wall", "-Wextra", *(extra_flags or []), "-shared", "-fPIC", SRC, "-o", lib + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
