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


def test_committed_traffic_is_plausible():
    """The counter record's bytes per launch stay within a few per cent of
    the algorithmic bytes for the streaming kernels, and at or above them
    for the tile kernels: a record that mixed in other workloads' launches
    (smaller grids) would fall below."""
    path = os.path.join(ROOT, "profiles", "hot_path_kernels_hbm_traffic.json")
    per = json.load(open(path))["per_launch"]
    streaming = {
        "logp_fwd_rows": 4.232e9,                  # 13926 active rows x 151936 x 2 B
        "logp_fwd_rows_entropy": 4.232e9,
        "logp_bwd_rows": 4.232e9 + 9.957e9,        # + 16384 x 151936 x 4 B written
        "log_softmax_rows": 4.232e9 + 9.957e9,
        "logp_bwd_rows_f32": 2 * 1.245e9,          # 2048 x 151936 x 4 B, read and written
    }
    for k, alg in streaming.items():
        moved = per[k]["read_bytes"] + per[k]["write_bytes"]
        assert 0.98 <= moved / alg <= 1.10, (k, moved, alg)
    minimum = {
        "linear_tiles_fwd_8192x128256x4096": 2 * (8192 + 128256) * 4096,
        "linear_tiles_fwd_2048x151936x5120": 2 * (2048 + 151936) * 5120,
        "linear_tiles_bwd_2048x151936x5120": 2 * (2048 + 151936) * 5120 + 4 * 2048 * 151936,
    }
    for k, alg in minimum.items():
        moved = per[k]["read_bytes"] + per[k]["write_bytes"]
        assert moved >= 0.98 * alg, (k, moved, alg)
