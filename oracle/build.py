"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles oracle.c with the host C compiler into liboracle.so beside it.
Plain IEEE arithmetic: no -ffast-math, so the oracle's fp64 results follow
the written order of operations.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force=True):
    """Compile liboracle.so; with force=False only when missing or stale."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
