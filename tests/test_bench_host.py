"""CPU tests of the benchmark's host helpers: reading the committed counter
summary must never fail the run (the round's benchmark line depends on it),
and the kernel-source hash that gates it is stable."""
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_line_parses_or_is_null():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    h = bench.kernel_source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert bench.kernel_source_hash() == h
    got = bench.traffic_from_profiles(h)  # the current sources: a figure or None
    assert got is None or got > 0
    assert bench.traffic_from_profiles("0" * 16) is None
    if os.path.exists(path):
        m = re.search(r"^traffic: .*\bsource_sha=(\S+)", open(path).read(), re.M)
        if m:  # the hash the counters were taken on gives their figure
            v = bench.traffic_from_profiles(m.group(1))
            assert v is not None and v > 0
