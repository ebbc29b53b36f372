"""Build the CPU oracle shared library (plain C99, gcc, OpenMP).

TEST INFRASTRUCTURE ONLY: the oracle is the checker of the GPU library, not a
part of it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ionn_oracle.c")
LIB = os.path.join(HERE, "libionn_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    """Compile ionn_oracle.c into libionn_oracle.so next to it; return the path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose="-v" in sys.argv))
