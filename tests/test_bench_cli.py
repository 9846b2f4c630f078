"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message before any device work, and the committed HBM-traffic
summary parses."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summary_parses():
    sys.path.insert(0, ROOT)
    import bench
    text = open(bench.TRAFFIC_FILE).read()
    assert "kernel_source_sha256" in text and "traffic_bytes_per_launch" in text
    t = bench.measured_traffic()
    # null only when the kernel sources changed after the counters were taken
    assert t is None or 1e9 < t < 1e13
    assert len(bench.kernel_source_sha()) == 64
