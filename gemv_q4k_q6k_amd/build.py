"""Build libgemvq.so in-tree with hipcc for gfx950.

    python -m gemv_q4k_q6k_amd.build

Compiles the kernels and the C ABI into one shared library next to this file.
Packed-FP32 instructions are disabled for all HIP code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgemvq.so")
ARCH = "gfx950"
SOURCES = ["gemvq_kernels.hip", "gemvq_abi.cpp"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out]


def build() -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgemvq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
