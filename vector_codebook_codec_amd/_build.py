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
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("api.hip", "calibrate.hip", "encode.hip", "plan.hip", "decode.hip", "matmul.hip",
                                                "metrics.hip", "polar.hip", "learn.hip")]
HEADERS = [os.path.join(CSRC, "qamw_device.h"), os.path.join(CSRC, "qamw_internal.h"),
           os.path.join(ROOT, "include", "qamw.h")]
LIB_PATH = os.path.join(PKG, "libqamw.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), flush=True)


# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
# device code is built as usual); for CPU-side checks of the C ABI's argument
# validation, with the sanitizer runtime preloaded into the checking process.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB_PATH = os.path.join(PKG, "libqamw_hostsan.so")


def build(verbose: bool = True, extra_flags=(), sanitize: bool = False) -> str:
    """Compile every HIP source (in parallel) and link libqamw.so; always recompiles.
    With sanitize, the host code is instrumented (ASan + UBSan) and the library
    goes to libqamw_hostsan.so instead."""
    from concurrent.futures import ThreadPoolExecutor

    flags = [*FLAGS, *extra_flags, *(SANITIZE_FLAGS if sanitize else [])]
    out = SANITIZED_LIB_PATH if sanitize else LIB_PATH
    tmpdir = tempfile.mkdtemp(prefix="qamw_build_", dir=PKG)
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[hipcc(), *flags, "-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp_lib = os.path.join(tmpdir, "libqamw.so")
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"]
        if sanitize:
            link += ["-fsanitize=address,undefined", "-shared-libsan"]
        _run([*link, "-o", tmp_lib, *objs], verbose)
        os.replace(tmp_lib, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


def sanitizer_runtime() -> str:
    """Path of the ASan runtime the sanitized library needs preloaded."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the HIP toolchain was not found")
    return path


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
