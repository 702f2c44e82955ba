"""bench.py's command line on the CPU: the multi-GPU request is refused with
a message and a non-zero status before any GPU work."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def test_bench_lists_its_legs():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for leg in ("decode", "prefill", "copy", "configs", "silu", "fused", "awq", "gptq"):
        assert leg in r.stdout
