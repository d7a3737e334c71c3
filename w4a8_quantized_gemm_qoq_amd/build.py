"""Build libqoq.so in-tree with hipcc for gfx950.

    python -m w4a8_quantized_gemm_qoq_amd.build

Compiles the HIP kernels, the host packer and the C-ABI shims into one shared
library next to this file.  No fast-math: the quantizers rely on IEEE FP32
division and round-half-to-even.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqoq.so")

SOURCES = ["status.cpp", "pack.cpp", "act_quant.hip", "gemm.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqoq.so)")


def build_command(out: str = LIB, arch: str = "gfx950") -> list[str]:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [
        hipcc(),
        f"--offload-arch={arch}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-fvisibility=hidden",
        "-Wall",
        "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-DQOQ_BUILD",
        "-o", out,
        *srcs,
    ]


def build(verbose: bool = False) -> str:
    """Compile libqoq.so; returns its path.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
