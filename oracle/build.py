"""Builds liboracle.so (plain C, gcc) beside this file.

Test infrastructure only: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only users of the oracle.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-Wno-unused-parameter", "-fPIC", "-shared",
        src, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
