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
    alg = ratio = kernels = None
    for line in open(os.path.join(ROOT, bench.COUNTERS[workload])):
        if line.startswith("# Algorithmic bytes per launch"):
            alg = float(line.split("=")[1].replace("B", "").replace(",", "").strip())
        if "traffic / algorithmic =" in line:
            ratio = float(line.split("=")[1])
        if line.startswith("kernel ="):
            kernels = line.split("=", 1)[1]
    assert alg is not None and ratio is not None
    assert abs(t / alg - ratio) < 1e-3
    if "merge" not in kernels:
        # one streaming split kernel: no input is read twice
        assert abs(t / alg - 1.0) < 0.01
    else:
        # a whole call: split records written and read back on top of the inputs
        assert t / alg > 1.0


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


def test_stamp_summary():
    """Per-workgroup stamps -> per-XCD summary: ends, spreads and the span had
    each XCD's share matched its own rate (harmonic mean of the XCD ends)."""
    import numpy as np
    n = 16
    st = np.zeros((n, 4), dtype=np.uint64)
    for w in range(n):
        x = w % 8
        st[w, 0] = 1000 + w            # starts 0.01 us apart (10 ns ticks)
        st[w, 1] = 1000 + 10000 + 100 * x + (w // 8)  # XCD x ends (100 + x) us after the first start
        st[w, 2] = x
        st[w, 3] = w
    s = bench.stamp_summary(st, 0.2)
    assert s["event_us"] == 200.0
    assert abs(s["start_spread_us"] - 0.15) < 1e-9
    ends = [100 + x + 0.01 for x in range(8)]
    assert abs(s["span_us"] - (107 + 0.01)) < 1e-9
    assert abs(s["xcd_end_min_max_us"][0] - 100.01) < 1e-9
    assert abs(s["balanced_span_us"] - 8 / sum(1 / e for e in ends)) < 1e-9
    assert s["xcd"]["3"]["workgroups"] == 2
    assert len(s["wg_duration_us"]) == n and s["wg_hw_id"][5] == 5


def test_event_stride():
    """Event-timed steps: one in four, but at least ten of the timed steps."""
    assert bench.event_stride(100) == 4
    assert bench.event_stride(200) == 4
    assert bench.event_stride(50) == 4
    assert bench.event_stride(30) == 3
    assert bench.event_stride(10) == 1
    assert bench.event_stride(1) == 1
    for K in range(1, 400):
        n = bench.event_stride(K)
        assert len(range(0, K, n)) >= min(K, 10)
