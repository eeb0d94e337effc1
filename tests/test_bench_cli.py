"""bench.py's command-line contract on the host (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_matches_its_schema():
    sys.path.insert(0, ROOT)
    import bench
    path = os.path.join(ROOT, "profiles", "hot_path_kernels_hbm_traffic.json")
    rec = json.load(open(path))
    assert set(rec) >= {"source_hash", "per_launch", "fetch_scale", "write_scale"}
    for v in rec["per_launch"].values():
        assert v["read_bytes"] >= 0 and v["write_bytes"] >= 0
    t = bench.measured_traffic()
    # either the committed counters belong to these sources, or they are not used
    assert (rec["source_hash"] == bench.source_hash()) == bool(t)
