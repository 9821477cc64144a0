"""bench.py's host-side pieces (CPU): the counter-traffic guard, the call-time
spread, the refusal of more than one GPU, and the committed counter
summaries that the bench reads."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("workload", sorted(bench.COUNTERS))
def test_committed_counters_match_the_sources(workload):
    """A committed counter summary that still hashes to the kernel sources it
    names gives the bench its traffic, within 1% of the algorithmic bytes
    recorded beside it (no re-reads).  A stale one is skipped: the bench
    then reports no traffic, as it should."""
    t = bench.counter_traffic(workload)
    if t is None:
        pytest.skip(f"{bench.COUNTERS[workload]} predates the current kernel sources")
    alg = None
    for line in open(os.path.join(ROOT, bench.COUNTERS[workload])):
        if line.startswith("# Algorithmic bytes per launch"):
            alg = float(line.split("=")[1].replace("B", "").replace(",", "").strip())
    assert alg is not None
    assert abs(t / alg - 1.0) < 0.01


def test_traffic_guard_rejects_changed_sources(tmp_path, monkeypatch):
    """A summary whose recorded hash does not match gives no traffic."""
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    summ = tmp_path / "k.counters.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.COUNTERS, "probe_workload", "k.counters.txt")
    good = bench.source_hash(["kernel.hip"])
    summ.write_text(f"# header\nsources = kernel.hip\nsource_sha256 = {good}\n"
                    "traffic_bytes_per_launch = 12345\n")
    assert bench.counter_traffic("probe_workload") == 12345.0
    src.write_text("// kernel v2\n")
    assert bench.counter_traffic("probe_workload") is None
    assert bench.counter_traffic("no_such_workload") is None


def test_spread():
    s = bench.spread([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s == {"median": 3.0, "p10": 1.0, "p90": 5.0, "calls": 5}
    assert bench.spread([7.0])["median"] == 7.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
