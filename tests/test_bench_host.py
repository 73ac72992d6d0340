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


class _ScriptedEvent:
    """Stands in for torch.cuda.Event: each (start, end) pair reports the next scripted time."""

    def __init__(self, script, **kw):
        self.script = script

    def record(self):
        pass

    def synchronize(self):
        pass

    def elapsed_time(self, end):
        return next(self.script)


def _settle_with(monkeypatch, times, min_ms, max_ms):
    import itertools

    import torch
    script = iter(itertools.chain(times, itertools.repeat(times[-1])))
    monkeypatch.setattr(torch.cuda, "Event", lambda **kw: _ScriptedEvent(script, **kw))
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a: None)
    calls = []
    bench.settle([lambda: calls.append(1)], "t", min_ms=min_ms, max_ms=max_ms)
    return bench.SETTLE_LOG["t"], len(calls)


def test_settle_waits_until_round_times_stop_falling(monkeypatch):
    """Round times that fall by 3% a round for 40 rounds and then hold: settling ends within two
    comparison windows of the plateau, not before it, and every queued round was launched."""
    W = bench.SETTLE_WINDOW
    falling = [10.0 * 0.97 ** i for i in range(40)]
    log, launched = _settle_with(monkeypatch, falling + [falling[-1]] * 100, min_ms=0.0, max_ms=1e9)
    read = log["rounds"] - 2  # rounds whose time was read; two more were still queued
    assert 40 + W <= read <= 40 + 2 * W + 1
    assert launched == log["rounds"]


def test_settle_stops_at_its_time_limit(monkeypatch):
    """Times that never stop falling (1.6% per window of 8 rounds, far from underflow within the
    cap): the wall-time cap ends the settle."""
    log, _ = _settle_with(monkeypatch, [1e6 * 0.998 ** i for i in range(200000)], min_ms=0.0, max_ms=30.0)
    assert 30.0 <= log["ms"] < 1000.0
