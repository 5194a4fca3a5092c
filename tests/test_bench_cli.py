"""bench.py's command line without a GPU: a multi-GPU request is refused
with a message and exit status 2 before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_is_refused():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=60, cwd=ROOT)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
        assert r.stdout == ""  # no JSON line for a run that did not happen
