"""bench.py's command line on the host: more than one GPU is refused with a message (no GPU touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_matches_gemm_sources():
    """The committed HBM-traffic record is only reported while the GEMM sources it was taken on are unchanged."""
    sys.path.insert(0, ROOT)
    import bench
    rec = bench.measured_traffic("igemm", "cfg2")
    import json
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        data = json.load(f)
    stored = data["igemm|cfg2"]["source_hash"]
    assert "bytes_per_call" in data["igemm|cfg2"]
    if stored == bench.source_hash():
        assert rec is not None and rec > 0
    else:
        assert rec is None
