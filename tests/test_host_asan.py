"""The library's host code under AddressSanitizer, on the CPU (no GPU).

The library is rebuilt with AddressSanitizer on its host side only (the
device code is compiled as usual but never runs here), and a C driver
(tests/cabi/host_asan.c), itself instrumented, exercises every host path that
returns before the first HIP call: status strings, the dispatch and split
choosers over 200000 seeded shapes, the buffer-window countdown up to
300 GiB, argument validation of the entry points and quick returns with
pointers that must never be dereferenced. Any out-of-bounds access, use after
free or similar error aborts the driver with a sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(ROOT, "precision_gemm_amd", "csrc", "sgemm.hip")
DRIVER = os.path.join(ROOT, "tests", "cabi", "host_asan.c")
INCLUDE = os.path.join(ROOT, "include")


def _tools():
    hip = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cc = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hip) and os.path.exists(cc)):
        pytest.skip("ROCm compilers not found")
    return hip, cc


def test_host_paths_under_address_sanitizer(tmp_path):
    hip, cc = _tools()
    lib = str(tmp_path / "libsgemm_asan.so")
    # The sanitizer applies to the host side of the build only.
    lib_cmd = [hip, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address",
               "-Xarch_host", "-fno-omit-frame-pointer",
               "-I", INCLUDE, SRC, "-o", lib]
    subprocess.run(lib_cmd, check=True, capture_output=True, timeout=900)
    exe = str(tmp_path / "host_asan")
    # The driver is host code from the start (a C program, no device code).
    drv_flags = ["-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
                 "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__"]
    drv_flags.append("-fsanitize=address")
    drv_cmd = [cc, *drv_flags, "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, DRIVER,
               "-o", exe, "-L", str(tmp_path), "-lsgemm_asan", "-Wl,-rpath," + str(tmp_path),
               "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
               "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(drv_cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    out = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "host checks: 0 failures" in out.stdout
    assert "AddressSanitizer" not in out.stderr
