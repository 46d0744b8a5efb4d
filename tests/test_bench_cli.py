"""bench.py's command line on the CPU: a request for more than one GPU ends
with a message and a non-zero status before anything touches a device."""
import os
import subprocess
import sys

from tests.conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run
