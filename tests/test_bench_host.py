"""Host-side checks of bench.py: the one-GPU guard and the traffic figure's provenance."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_record_matches_sources_or_is_withheld(monkeypatch):
    for part in ("prefill", "decode"):
        rec, src = bench.traffic_record(part)
        if rec is not None:  # a committed profile of exactly these sources
            assert rec["source_sha256_16"] == bench.source_digest(part)
            # each of the three is rounded to whole bytes on its own
            assert abs(rec["bytes_per_launch"] - rec["read_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 1
            assert src.startswith("profiles" + os.sep)
    # once a kernel source differs from the profiled one, no traffic figure is reported
    monkeypatch.setattr(bench, "source_digest", lambda part: "0" * 16)
    for part in ("prefill", "decode"):
        rec, why = bench.traffic_record(part)
        assert rec is None and ("other sources" in why or "no counter profile" in why)
