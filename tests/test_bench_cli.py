"""bench.py's option checks, which end the run before any GPU work."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("args, text", [
    (("--launch-per-group", "--batch", "2"), "batch L = 1"),
    (("--format", "mxfp4", "--sf-layout", "blocked"), "row-major scales only"),
    (("--batch", "2", "--format", "mxfp4"), "NVFP4 row-major scales only"),
])
def test_unsupported_combinations_are_refused(args, text):
    r = run_bench(*args)
    assert r.returncode == 2, r.stderr
    assert text in r.stderr
