"""bench.py's command line on the CPU: it measures one GPU and says so for more."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120)
        assert p.returncode == 2
        assert "one GPU" in p.stderr and f"--gpus {n}" in p.stderr
        assert p.stdout == ""


def test_help_lists_the_benchmark_modes():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 0
    for flag in ("--steps", "--warmup", "--config", "--format", "--encode", "--pipeline",
                 "--fused", "--fused-gemm", "--tokens", "--copy-bytes", "--no-cpu-baseline"):
        assert flag in p.stdout
