"""The committed HBM-traffic record that bench.py reports as roofline.traffic: well formed, calibrated against the
copy kernel, and used only while the sources it hashes are unchanged."""
import hashlib
import json
import os
import shutil

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REC = os.path.join(ROOT, "profiles", "traffic_batch64_decode.json")


def _sha(root, paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(root, p), "rb").read())
    return h.hexdigest()[:16]


def test_record_covers_the_timed_stages():
    rec = json.load(open(REC))
    # on a 1 GiB device copy FETCH_SIZE counts half the bytes read and WRITE_SIZE all the bytes written
    assert abs(rec["fetch_factor"] - 2.0) < 0.01 and abs(rec["write_factor"] - 1.0) < 0.01
    for stage, kernels in bench.STAGE_KERNELS.items():
        for k in kernels:
            e = rec["kernels"][k]
            assert e["read_bytes"] > 0 and e["write_bytes"] >= 0
            for src in e["sources"]:
                assert os.path.exists(os.path.join(ROOT, src)), src


def test_traffic_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    rec = json.load(open(REC))
    fresh = all(_sha(ROOT, rec["kernels"][k]["sources"]) == rec["kernels"][k]["sha256_16"]
                for k in bench.STAGE_KERNELS["attend"])
    want = int(sum(rec["kernels"][k]["read_bytes"] + rec["kernels"][k]["write_bytes"]
                   for k in bench.STAGE_KERNELS["attend"]))
    assert bench.measured_traffic("attend") == (want if fresh else None)
    # a copy of the tree whose attention source differs by one byte: the record no longer applies
    src = rec["kernels"][bench.STAGE_KERNELS["attend"][0]]["sources"]
    for p in src + ["profiles/traffic_batch64_decode.json"]:
        os.makedirs(tmp_path / os.path.dirname(p), exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), tmp_path / p)
    with open(tmp_path / src[0], "ab") as f:
        f.write(b"\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("attend") is None
