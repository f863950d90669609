"""Host-side contract of bench.py: one GPU only, with a clear message."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_defaults_finish_quickly():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert (a.gpus, a.workload) == (1, "3a")
    assert a.steps >= 20 and a.warmup >= 3          # median over >= 20 reps after 3 warm-ups
    assert 10 <= a.cpu_seconds <= 30                # bounded CPU-baseline sample
