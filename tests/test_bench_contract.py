"""bench.py's host-side contract (no GPU needed): a request for more than one
GPU is refused with a message and exit status 2, and the recorded HBM
traffic file is well formed."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run


def test_recorded_traffic_lines_are_well_formed():
    lines = [ln for ln in open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")) if ln.strip()
             and not ln.startswith("#")]
    assert lines
    for ln in lines:
        workload, sha, fetch, write = ln.split()
        assert re.fullmatch(r"[a-z0-9_]+", workload)
        assert re.fullmatch(r"[0-9a-f]{64}", sha)
        assert int(fetch) > 0 and int(write) > 0
