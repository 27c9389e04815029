"""Build the oracle's C core (``oracle/_gs_oracle.so``) with gcc.

Test infrastructure: the library built here is what the tests compare the
product against, never part of the product path. Plain IEEE float64 (no
fast-math, no contraction) so the arithmetic is exactly what the source says.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "gs_oracle.c")
OUT = os.path.join(HERE, "_gs_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(OUT) and os.path.getmtime(OUT) >= os.path.getmtime(SRC):
        return OUT
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(force="--lazy" not in sys.argv))
