"""Build libqoq.so in-tree with hipcc for gfx950.

    python -m w4a8_quantized_gemm_qoq_amd.build

Compiles the HIP kernels, the host packer and the C-ABI shims into one shared
library next to this file (one object per source, compiled in parallel under
_build/, then linked).  No fast-math: the quantizers rely on IEEE FP32
division and round-half-to-even.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqoq.so")
# Written next to the library by build(): the hash of the sources and flags it
# was built from.  load_library() refuses a library whose record is missing or
# differs from the sources in the tree.
HASH_FILE = LIB + ".srchash"

SOURCES = ["status.cpp", "pack.cpp", "transforms.cpp", "act_quant.hip", "kv4.hip", "gemm_w4.hip", "gemm_w8.hip", "gemm_sat.hip"]
OBJDIR = os.path.join(PKG, "_build")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqoq.so)")


def compile_flags(arch: str = "gfx950") -> list[str]:
    return [
        f"--offload-arch={arch}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        "-Wall",
        "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-DQOQ_BUILD",
    ]


def source_hash(arch: str = "gfx950") -> str:
    """SHA-256 of every file under csrc/ and include/ (bytes, sorted by name)
    and of the compile flags: what the library is built from."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(os.path.relpath(path, ROOT).encode() + b"\0")
                with open(path, "rb") as f:
                    h.update(f.read())
    h.update("\0".join(compile_flags(arch)).replace(ROOT, "").encode())
    return h.hexdigest()


def build_commands(out: str = LIB, arch: str = "gfx950") -> tuple[list[list[str]], list[str]]:
    """One compile command per source (independent, run in parallel), then the link."""
    flags = compile_flags(arch)
    objs, compiles = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        objs.append(obj)
        compiles.append([hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    link = [hipcc(), f"--offload-arch={arch}", "-shared", "-fPIC", "-o", out, *objs]
    return compiles, link


def build(verbose: bool = False) -> str:
    """Compile libqoq.so; returns its path.  Always recompiles."""
    os.makedirs(OBJDIR, exist_ok=True)
    digest = source_hash()
    if os.path.exists(HASH_FILE):
        os.remove(HASH_FILE)
    tmp = LIB + ".tmp"
    compiles, link = build_commands(tmp)
    procs = []
    for cmd in compiles:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((cmd[-3], p.returncode, out))
    if failed:
        for src, rc, out in failed:
            sys.stderr.write(f"{src}: exit code {rc}\n{out}")
        raise RuntimeError(f"hipcc failed on {', '.join(f[0] for f in failed)}")
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    with open(HASH_FILE, "w") as f:
        f.write(digest + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
