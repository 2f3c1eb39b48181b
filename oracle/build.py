"""Builds liboracle.so (plain C, gcc) beside this file.

Test infrastructure only: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only users of the oracle.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build, loaded instead of LIB
# when SPEC_ORACLE_LIB points at it (tests/run_sanitizers.sh)
SAN_LIB = os.path.join(os.path.dirname(HERE), "_build", "sanitize", "liboracle.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    out = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"] if sanitize else []
    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-Wno-unused-parameter", "-fPIC", "-shared", *san,
        src, "-o", out + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
