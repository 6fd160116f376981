"""bench.py's command line on the CPU: it runs on one GPU only, and says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_traffic_summaries_parse():
    """The counter summaries bench.py reads carry the fields it needs, and their
    traffic is within a few percent above the algorithmic bytes they state."""
    sys.path.insert(0, ROOT)
    import bench
    for path in (bench.TRAFFIC_SUMMARY, bench.TRAFFIC_SUMMARY_FP8):
        kv = {}
        with open(os.path.join(ROOT, path)) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].strip().split(": ", 1)
                    kv[k] = v
        alg, traffic = int(kv["algorithmic_bytes_per_launch"]), int(kv["traffic_bytes_per_launch"])
        assert 1.0 <= traffic / alg < 1.1, path
        assert len(kv["source_sha256"]) == 64
