"""bench.py's host-side refusal of more than one GPU: it ends with status 2
and one JSON line naming the reason, before any GPU work."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    return r.returncode, json.loads(r.stdout.strip().splitlines()[-1])


def test_more_than_one_gpu_is_refused():
    code, line = _run("--gpus", "2")
    assert code == 2 and line["n_gpus"] == 2 and "one GPU" in line["error"]

