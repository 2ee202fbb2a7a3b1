"""tests/test_abi.py against a build of the library whose host code (the C
ABI's argument checks, sizes and workspace arithmetic) is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built as
usual and no kernel runs.  The ASan runtime is preloaded into a child pytest
(after any preload the environment already names).  Opt in with
QAMW_HOSTSAN=1: the build recompiles every source (about two minutes)."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(os.environ.get("QAMW_HOSTSAN") != "1", reason="opt in with QAMW_HOSTSAN=1 (a full rebuild)")
def test_abi_under_host_sanitizers():
    sys.path.insert(0, ROOT)
    from vector_codebook_codec_amd import _build

    lib = _build.build(verbose=False, sanitize=True)
    preload = _build.sanitizer_runtime()
    if os.environ.get("LD_PRELOAD"):
        preload += ":" + os.environ["LD_PRELOAD"]
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", QAMW_LIBRARY=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(HERE, "test_abi.py")], env=env, cwd=ROOT, capture_output=True, text=True,
                         timeout=900)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout and "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
