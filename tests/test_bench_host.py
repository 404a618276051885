"""Host-side checks of bench.py: the one-GPU refusal, the bulk-quantize byte accounting and the
counter-traffic record."""
import json
import os
import subprocess
import sys

import pytest

from oracle import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("gpus", [2, 8])
def test_more_than_one_gpu_is_refused(gpus):
    """--gpus above 1 exits with status 2 and one JSON line that says why, before any GPU work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(gpus)],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == gpus and "one GPU" in line["error"]


@pytest.mark.parametrize("kb,kq,vb", [(2, 1, 3), (3, 1, 4), (0, 1, 3), (1, 1, 2), (4, 0, 4)])
def test_bulk_bytes_match_the_layout(kb, kq, vb):
    """Bulk quantize moves, per token and head, a bf16 key and value in (2 x 128 x 2 bytes) and
    the packed record out (the layout's bytes per token)."""
    B, Hkv, n = 3, 2, 1000
    assert bench.bulk_bytes(B, Hkv, n, kb, kq, vb) == B * Hkv * n * (512 + layout.bytes_per_token(kb, kq, vb)["total"])


def test_counter_traffic_only_for_the_sources_it_was_taken_on(monkeypatch):
    """The HBM bytes of the committed counter summary are reported for the workloads it covers
    while the attention sources hash to the digest recorded with them, and are None otherwise
    (so a changed kernel never carries stale counter figures)."""
    rec = json.load(open(bench.TRAFFIC_FILE))
    digest = bench.attend_sources_sha256()
    for e in rec["entries"]:
        assert abs(e["hbm_bytes_per_launch"] - e["fetch_bytes_per_launch"] - e["write_bytes_per_launch"]) <= 1
        assert e["hbm_bytes_per_launch"] >= e["algorithmic_bytes_per_launch"]
        expect = float(e["hbm_bytes_per_launch"]) if e["source_sha256"] == digest else None
        assert bench.measured_traffic(e["workload"], e["preset"]) == expect
    assert bench.measured_traffic("no_such_workload", "turbo3") is None
    monkeypatch.setattr(bench, "attend_sources_sha256", lambda: "0" * 64)
    for e in rec["entries"]:
        assert bench.measured_traffic(e["workload"], e["preset"]) is None
