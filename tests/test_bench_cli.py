"""The benchmark's command line on a machine without a GPU: more than one GPU
is refused with a message (one GPU is all the codec's benchmark uses)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)
    assert not res.stdout.strip().startswith("{")      # no result line
