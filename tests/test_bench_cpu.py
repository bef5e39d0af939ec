"""bench.py's command-line contract, on the CPU: more than one GPU is refused
with a message before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    pr = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                        capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert pr.returncode != 0
    assert "exactly one GPU" in (pr.stdout + pr.stderr)
    assert not pr.stdout.strip().startswith("{")      # no JSON line
