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
LIB_ASAN = os.path.join(HERE, "liboracle_asan.so")


def build(force=True, asan=False):
    """Compile liboracle.so; with force=False only when missing or stale.
    asan=True builds liboracle_asan.so with AddressSanitizer (for test runs
    with the ASan runtime preloaded; load it by setting ORACLE_LIB)."""
    out = LIB_ASAN if asan else LIB
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    san = ["-fsanitize=address", "-fno-omit-frame-pointer", "-g"] if asan else []
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall"] + san + [
           "-o", out + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    import sys
    print(build(asan="--asan" in sys.argv[1:]))
