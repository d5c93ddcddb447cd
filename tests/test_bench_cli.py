"""bench.py's command line on the CPU: asking for more than one GPU exits with status 2 and a message
saying the library runs on one GPU, before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert run.returncode == 2
    assert "one GPU" in run.stderr
    assert run.stdout == ""
