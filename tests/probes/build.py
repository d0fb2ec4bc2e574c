"""Build the test-only MFMA probe library (tests/probes/libprobes.so) for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_probe.hip")
LIB = os.path.join(HERE, "libprobes.so")


def build(out: str = LIB) -> str:
    sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
    from precision_gemm_amd import _build
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([_build.hipcc(), *_build.flags(), SRC, "-o", tmp], check=True, cwd=HERE)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
