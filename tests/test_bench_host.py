"""Host-side checks of bench.py: the one-GPU rule, the counter-record logic
behind roofline.traffic, and the committed record's own arithmetic."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_reported_only_for_matching_source(tmp_path, monkeypatch):
    import bench
    rec = {"kernel_source_sha256": bench.kernel_source_hash(), "bytes_per_launch": 123.0}
    path = tmp_path / "rec.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.traffic_from_record()[0] == 123.0
    rec["kernel_source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    value, why = bench.traffic_from_record()
    assert value is None and "changed" in why
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.json"))
    assert bench.traffic_from_record()[0] is None


def test_committed_counter_record_is_consistent():
    """The record's totals follow from its raw counters and copy calibration,
    and its algorithmic bytes are those of the dense 8k workload: Q, K, V read
    once (bf16), O written once (bf16) and lse once (fp32)."""
    import bench
    with open(bench.TRAFFIC_RECORD) as f:
        rec = json.load(f)
    B, H, N, d = 8, 32, 8192, 128
    assert rec["algorithmic_read_bytes"] == 3 * B * H * N * d * 2
    assert rec["algorithmic_write_bytes"] == B * H * N * d * 2 + B * H * N * 4
    gib_kib = (1 << 30) / 1024
    assert rec["fetch_scale"] == pytest.approx(gib_kib / rec["copy_fetch_kib_per_GiB"], rel=1e-9)
    assert rec["write_scale"] == pytest.approx(gib_kib / rec["copy_write_kib_per_GiB"], rel=1e-9)
    read = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"]
    write = rec["write_kib_per_dispatch"] * 1024 * rec["write_scale"]
    assert rec["read_bytes_per_launch"] == pytest.approx(read, rel=1e-9)
    assert rec["write_bytes_per_launch"] == pytest.approx(write, rel=1e-9)
    assert rec["bytes_per_launch"] == pytest.approx(read + write, rel=1e-9)
    for cmd in rec["commands"]:
        assert "bench.py" in cmd and "_work" not in cmd
