"""Build libqamw.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m vector_codebook_codec_amd._build

The library lands next to this file so that it travels with the source tree.
Packed FP32 instructions are disabled for the whole build
(-target-feature -packed-fp32-ops); kernels use scalar fp32 FMA/min.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "qamw_kernels.hip")]
HEADERS = [os.path.join(PKG, "csrc", "qamw_device.h"), os.path.join(ROOT, "include", "qamw.h")]
LIB_PATH = os.path.join(PKG, "libqamw.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_command(out: str) -> list:
    return [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-o", out, *SOURCES,
    ]


def build(verbose: bool = True) -> str:
    """Compile every HIP source into libqamw.so (always recompiles)."""
    fd, tmp = tempfile.mkstemp(prefix="libqamw.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "packed-fp32-ops"
        msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        if msgs and verbose:
            print("\n".join(msgs), flush=True)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
