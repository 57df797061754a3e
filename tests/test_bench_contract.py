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


def test_negative_head_count_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--heads", "-1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--heads" in r.stderr
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


def test_parity_record_from_the_cpu_baseline_leg():
    """The bench's parity record, fed the oracle's own results as the GPU
    side (O rounded to bf16), passes with no mask mismatch; a row with one
    block swapped for a low-scoring one counts as a mismatch that is not a
    near-tie, and fails the record."""
    import numpy as np
    import lcsa_inputs as li
    import oracle
    name = "small_edges"
    desc = li.CONFIGS[name]
    inp = li.generate(desc, seed=3)
    g = oracle.geometry(desc)
    q, k, v = (li.bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    rp, ci, s = oracle.select(g, q, k)
    o, lse = oracle.attend(g, q, k, v, rp, ci)
    o_bf16 = li.bf16_bits_to_f32(li.f32_to_bf16_bits(o.astype(np.float32)))
    base, par = bench.cpu_baseline(name, desc, inp, oracle.useful_flops(g, rp),
                                   (rp, ci, o_bf16, lse.astype(np.float32)), runs=1)
    assert par["pass"] and par["mask_rows_differing"] == 0
    assert par["attend_elements"] == o.size and par["attend_cosine"] > 0.9999
    assert base["kind"] == "oracle" and base["cores"] >= 1 and len(base["attend_s_runs"]) == 1
    # swap row 0's lowest kept block for the window block with the lowest score
    ci2 = ci.copy()
    e = oracle.window(g, 0)
    worst = int(e[np.argmin(s[0, 0, 0, e])])
    row = ci2[rp[0]:rp[1]]
    assert worst not in row
    row[np.argmin(s[0, 0, 0, row])] = worst
    ci2[rp[0]:rp[1]] = np.sort(row)
    mism, ties = bench._mask_parity(g, oracle.window, rp, ci, s, rp, ci2)
    assert mism == [0] and ties == 0
