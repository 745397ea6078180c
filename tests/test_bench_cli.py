"""bench.py's command-line contract on the host: a run on more than one GPU is refused with one
JSON line and exit status 2 before any device work; the traffic figure is looked up only for a
known kernel kind."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1 and "error" in json.loads(lines[0])


def test_traffic_lookup_only_for_known_kinds():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic("no such kernel kind") is None
    h = bench.kernel_source_hash()
    assert len(h) == 64 and all(c in "0123456789abcdef" for c in h)
