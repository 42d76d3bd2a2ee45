"""bench.py's command-line contract and its HBM-traffic lookup, on the CPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_traffic_is_reported_only_for_the_sources_it_was_counted_on(monkeypatch):
    """profiles/pmc_traffic.json carries a digest of the library sources:
    the byte counts are used while it matches and dropped (None) once the
    sources change."""
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as f:
        rec = json.load(f)
    k = rec["kernels"]["score_lore"]
    expect = int(round((k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"]) * 1024))
    monkeypatch.setattr(bench, "_csrc_digest", lambda: rec["source_digest"])
    assert bench.measured_traffic("score_lore") == expect
    # the selection spans both of its kernels
    parts = [rec["kernels"][p] for p in ("topb_local", "topb_select")]
    both = sum((p["fetch_kib"] * rec["fetch_scale"] + p["write_kib"] * rec["write_scale"]) * 1024
               for p in parts)
    assert bench.measured_traffic("topb") == int(round(both))
    assert bench.measured_traffic("no_such_kernel") is None
    monkeypatch.setattr(bench, "_csrc_digest", lambda: "0" * 64)
    assert bench.measured_traffic("score_lore") is None
