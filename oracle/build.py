"""Build the C oracle (oracle/kla_ref.c) into oracle/libkla_ref.so with gcc.

TEST INFRASTRUCTURE: the C oracle is loaded only by tests, smoke() and the
bench's cpu_baseline leg. No -ffast-math: the oracle keeps IEEE double semantics.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kla_ref.c")
LIB = os.path.join(HERE, "libkla_ref.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
