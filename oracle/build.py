"""Build the C part of the oracle (test infrastructure) with gcc.

The oracle is compiled for the baseline x86-64 target (no -march=native), so
that a library built in one container runs on any x86-64 host.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "recurrent.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
