"""Builds the CPU oracle (plain C, gcc) into oracle/libfp4q_oracle.so.

Test infrastructure only: the product library never links or loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4q_oracle.c")
LIB = os.path.join(HERE, "libfp4q_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc -O2 (C99, no fast-math) and return the path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
