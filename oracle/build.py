"""Build the CPU oracle library (plain C, gcc, OpenMP, no FMA contraction).

Test infrastructure only: the oracle is the checker, never the product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cp_oracle.c")
LIB = os.path.join(HERE, "liborc.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
