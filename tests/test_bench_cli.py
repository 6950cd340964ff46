"""bench.py's command line on the CPU: a run on more than one GPU is refused
before anything touches a device (this build measures one GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")  # no measurement line
