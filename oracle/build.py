"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off: every product and sum is rounded as written (no FMA
    # fusion), so the oracle's arithmetic is exactly what the source says.
    cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
