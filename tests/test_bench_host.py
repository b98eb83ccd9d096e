"""bench.py's host-side contract, on the CPU: it measures one GPU only and says
so (exit status 2) when asked for more, before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""
