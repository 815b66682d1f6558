"""CPU checks of the benchmark's contract: one GPU only, and the HBM-traffic figure is taken from
the committed counter summary only while it was measured on the current forward sources."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 1" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.lstrip().startswith("{")


def test_traffic_is_read_only_for_matching_sources(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["hbm_bytes_per_launch"] > 0
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    # a summary taken on these sources is used ...
    p.write_text(json.dumps(dict(t, kernel_source_sha256_16=bench.source_hash(bench.FWD_SRC))))
    assert bench.load_traffic() == t["hbm_bytes_per_launch"]
    # ... one of other sources is ignored (traffic reported as null), as is a missing file
    p.write_text(json.dumps(dict(t, kernel_source_sha256_16="0" * 16)))
    assert bench.load_traffic() is None
    p.unlink()
    assert bench.load_traffic() is None
