"""Build the fp64 CPU oracle (test infrastructure) with gcc.

    python oracle/build.py

writes oracle/libssd_oracle.so. -ffp-contract=off keeps every multiply and
add a separate IEEE operation, so a run continued from a carried state
repeats the exact operation sequence of an unbroken run.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "libssd_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
