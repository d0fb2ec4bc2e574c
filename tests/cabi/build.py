"""Build the test-only C caller of libsgemm (tests/cabi/sgemm_client).

A plain C11 program compiled with gcc against include/sgemm.h and the HIP
runtime's C API, linked to the in-tree libsgemm.so through a relative rpath so
that the tree can be moved as a whole.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "sgemm_client.c")
EXE = os.path.join(HERE, "sgemm_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = EXE) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "precision_gemm_amd"), "-lsgemm",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../precision_gemm_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
