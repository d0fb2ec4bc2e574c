"""Compile the CPU oracle (plain C, gcc) into ``oracle/liboracle_sgemm.so``.

Test infrastructure: the flags keep every double operation separately rounded
(no contraction into fused multiply-add, no fast-math reassociation).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sgemm_oracle.c")
LIB = os.path.join(HERE, "liboracle_sgemm.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-std=c99", "-Wall", "-Wextra", "-pthread"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
