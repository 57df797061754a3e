"""Host-side checks of bench.py: it refuses more than one GPU before touching
torch or a device, and the HBM traffic it reports comes only from a counter
record taken on the current attention kernel source."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_record_keyed_by_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "attend.hip"
    src.write_text("kernel v1\n")
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"first_768x1280": {"attend_src_sha256": bench._src_sha(str(src)),
                                                  "bytes_per_launch": 1234}}))
    monkeypatch.setattr(bench, "ATTEND_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench._traffic("first_768x1280") == 1234
    assert bench._traffic("stream_768x1280") is None      # no record for that workload
    src.write_text("kernel v2\n")                          # kernel changed since the counters
    assert bench._traffic("first_768x1280") is None


def test_committed_traffic_record_is_well_formed():
    rec = json.load(open(bench.TRAFFIC_FILE))
    entry = rec["first_768x1280"]
    assert entry["kernel"].startswith("attend_fwd_kernel")
    assert len(entry["attend_src_sha256"]) == 64
    # at least the algorithmic Q + K + V + O bytes of one launch (4 x 70.8 MB)
    assert entry["bytes_per_launch"] >= 4 * 23040 * 12 * 128 * 2
