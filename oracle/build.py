"""Build the oracle's shared library with gcc (test infrastructure only).

The oracle is plain C: ``gcc -O2 -fopenmp``, no fast-math, so that every
double and float operation is IEEE round-to-nearest as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "moe_oracle.c")
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
        src, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
