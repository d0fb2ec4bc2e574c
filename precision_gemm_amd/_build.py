"""Build the HIP library ``libsgemm.so`` for gfx950 with hipcc.

Every kernel is compiled with packed-FP32 instruction selection switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``): the FP32 work of this
library runs on MFMA, and plain float code must not be turned into packed
v_pk_* FP32 arithmetic on this platform.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "sgemm.hip")
LIB = os.path.join(PKG, "libsgemm.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsgemm)")


def flags(save_temps_dir: str | None = None) -> list[str]:
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", INCLUDE]
    if save_temps_dir:
        f += ["--save-temps"]
    return f


def build(out: str = LIB, save_temps_dir: str | None = None) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(save_temps_dir), SRC, "-o", tmp]
    subprocess.run(cmd, check=True, cwd=save_temps_dir or PKG)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(save_temps_dir=sys.argv[1] if len(sys.argv) > 1 else None))
