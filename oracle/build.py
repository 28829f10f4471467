"""Compile the C oracle (test infrastructure; see oracle/__init__.py).

Only tests, the smoke check and the CPU-baseline leg of the benchmark use
the oracle.  It is built with plain gcc, no fast-math and no contraction,
so every butterfly add and subtract is one IEEE operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(force=True):
    """Compile oracle.c into liboracle.so next to it; returns the path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-D_POSIX_C_SOURCE=200809L", "-Wall", "-Wextra", "-shared", "-fPIC",
           SRC, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle())
