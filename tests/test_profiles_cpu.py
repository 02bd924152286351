"""The committed rocprofv3 summaries under profiles/ agree with the sources and with themselves.

bench.py attaches a counter-measured HBM traffic figure to a workload's roofline only while the
kernel sources hash to the value stored beside it; these checks make a stale record fail here
instead of silently turning into null. Each record's stored bytes per call must also be the
sum of its own table (HBM read + write MB per kernel), and every summary must give the
rocprofv3 command that produced it.
"""
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC_RECORDS))
def test_traffic_record_current(workload):
    got = bench.measured_traffic(workload)
    assert got is not None, f"{workload}: traffic record missing or its kernel sources changed since"
    assert got > 0


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC_RECORDS))
def test_traffic_record_matches_its_table(workload):
    _, record = bench.TRAFFIC_RECORDS[workload]
    text = open(record).read()
    read_mb = write_mb = 0.0
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        # | kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM read (MB) | HBM write (MB) |
        if len(cells) == 6 and cells[0].startswith("`"):
            read_mb += float(cells[4])
            write_mb += float(cells[5])
    assert read_mb > 0
    total = bench.measured_traffic(workload)
    # per-kernel figures are rounded to 0.1 MB
    n_rows = text.count("\n| `")
    assert abs(total / 1e6 - (read_mb + write_mb)) <= 0.05 * 2 * n_rows + 1e-6


def test_every_summary_names_its_command():
    names = sorted(f for f in os.listdir(PROFILES) if f.endswith((".md", ".txt")))
    assert names
    for name in names:
        text = open(os.path.join(PROFILES, name)).read()
        assert re.search(r"rocprofv3 .*--( |.*-- )python3? bench\.py", text), name
