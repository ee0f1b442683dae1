"""Address and undefined-behaviour sanitizer runs of the host code (CPU only).

Two test programs under tests/sanitize/, each built here with the sanitizers
on and run to completion:

* the C oracle: every function on exact-size heap buffers over shapes from one
  super-block to K = 32768, with 1 and 2 OpenMP threads (gcc,
  -fsanitize=address,undefined);
* the C-ABI library's host code: every entry point with arguments its checks
  must reject (the status codes are asserted; a rejected call makes no HIP
  call), and the launch planner of every kind over a grid of shapes through
  the geometry hook.  hipcc instruments the host pass only; device code is
  built as for the product.

A sanitizer report aborts the program (-fno-sanitize-recover=all), so a zero
exit status means a clean run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, (cmd, p.returncode, p.stdout[-3000:], p.stderr[-3000:])
    return p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-ffp-contract=off",
         os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
         "-o", exe, "-lm"])
    out = run([exe], env=dict(SAN_ENV, OMP_NUM_THREADS="2"), timeout=600)
    assert "clean" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "gemv_q4k_q6k_amd", "csrc")
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-x", "hip",
         os.path.join(csrc, "gemvq_kernels.hip"), os.path.join(csrc, "gemvq_abi.cpp"),
         os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe], cwd=str(tmp_path))
    out = run([exe], env=SAN_ENV, timeout=600)
    assert "0 failures" in out
