"""Builds the C oracle into oracle/liboracle.so.

Test infrastructure: plain gcc, -O2, fp contraction off, no fast-math, no
intrinsics, single thread.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["moe_oracle.c", "cache_sim.c"]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp"]
    cmd += [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = SOURCES + ["moe_oracle.h"]
    return any(os.path.getmtime(os.path.join(HERE, d)) > t for d in deps)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
