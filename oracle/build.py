"""Build the oracle's shared library with the host C compiler.

Test infrastructure only: the oracle is never part of the GPU library.
Usage: python -m oracle.build   (or call build()).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mmac_oracle.c")
LIB = os.path.join(HERE, "libmmac_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile mmac_oracle.c with gcc -O2 -fopenmp (no -ffast-math: the sum order is fixed)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
