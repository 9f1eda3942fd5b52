"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libqlin is compiled with the sanitizers on its host side only
(device code is unchanged), linked into tests/host_sanitizer/validation_driver.cpp,
and run without a GPU: the driver calls every entry point with arguments
that validation must reject (including sizes whose products overflow 64 bits)
and with empty batches.  Any sanitizer report or unexpected status fails.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "outlier_aware_bit_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_sanitizer", "validation_driver.cpp")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

# Host-side sanitizer flags for hipcc: each one behind -Xarch_host, so device
# code is compiled as usual.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
LINK_SAN = ["-fsanitize=address", "-fsanitize=undefined"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_validation_under_host_sanitizers(tmp_path):
    out = str(tmp_path)
    common = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-I", INCLUDE]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src)[:-4] + ".o")
        _run([HIPCC, "--offload-arch=gfx950", *common, *HOST_SAN, "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", CSRC, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(out, "driver.o")
    _run([CLANG, *common, *LINK_SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-c", DRIVER,
          "-o", drv])
    exe = os.path.join(out, "validation_driver")
    _run([CLANG, *LINK_SAN, "-o", exe, drv, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib")])

    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    log = r.stdout + r.stderr
    if r.returncode == 77:
        pytest.skip("a GPU is visible: the driver checks host code only")
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
    assert r.returncode == 0, log
    assert " 0 failures" in log, log
    shutil.rmtree(out, ignore_errors=True)
