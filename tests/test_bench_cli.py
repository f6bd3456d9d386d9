"""CPU checks of bench.py's command line: the path runs on one GPU, so any
other GPU count is refused with a message before anything is built or run."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, r.stderr
        msg = json.loads(r.stdout.strip().splitlines()[-1])
        assert "one GPU" in msg["error"] and "--gpus must be 1" in msg["error"]


def test_cpu_model_is_read_from_the_host():
    sys.path.insert(0, ROOT)
    import bench
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
