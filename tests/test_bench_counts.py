"""The FLOP convention of bench.py: visible (query, key) pairs of a chunk pair,
counted in closed form, against brute-force enumeration on small chunks."""

import importlib.util
import os

import pytest

import oracle

_spec = importlib.util.spec_from_file_location(
    "bench", os.path.join(os.path.dirname(os.path.dirname(__file__)), "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _brute(a, c_, chunk, window):
    n = 0
    for i in range(chunk):
        for j in range(chunk):
            d = (a * chunk + i) - (c_ * chunk + j)
            if d >= 0 and (window <= 0 or d < window):
                n += 1
    return n


@pytest.mark.parametrize("p,chunk,window", [(4, 8, 0), (5, 6, 3), (4, 8, 8), (6, 5, 12), (3, 7, 1)])
def test_visible_pairs_match_enumeration(p, chunk, window):
    items = (oracle.window_schedule(p, chunk, window)[0] if window > 0
             else oracle.balanced_schedule(p)[0])
    for it in items:
        assert bench.visible_pairs(it, chunk, window) == _brute(it[2], it[3], chunk, window), it


def test_causal_pair_counts():
    assert bench.pairs_of(0, 32768) == 32768 * 32769 // 2
    assert bench.pairs_of(1, 32768) == 32768 ** 2


@pytest.mark.parametrize("p,chunk,window,g", [(4, 8, 3, 2), (5, 6, 7, 6), (3, 7, 1, 1), (6, 5, 12, 3)])
def test_global_visible_pairs_sum_to_the_masked_pairs(p, chunk, window, g):
    """Summed over the global-window schedule, the counted pairs are exactly
    the (query, key) pairs the global-token mask keeps."""
    items = oracle.global_window_schedule(p, chunk, window, g)[0]
    got = sum(bench.visible_pairs(it, chunk, window, g) for it in items)
    want = sum(1 for i in range(p * chunk) for j in range(i + 1) if i - j < window or j < g)
    assert got == want
    for it in items:
        if it[3] == -1:  # the global item: every causal key of the prefix
            assert bench.visible_pairs(it, chunk, window, g) == sum(
                min(g, it[2] * chunk + i + 1) for i in range(chunk))


def test_traffic_summary_is_used_only_for_its_sources_and_workload():
    """The committed HBM-traffic summary is reported for a kernel only when it
    was taken on that kernel's current sources, and never for another
    workload; where it is reported its parts add up."""
    import json
    doc = json.load(open(bench.TRAFFIC_FILE))
    for name in bench.KERNEL_SOURCES:
        entry = doc["kernels"].get(name)
        t = bench.traffic_of(name, 1, doc["workload"])
        if entry is None or entry["source_digest"] != bench.source_digest(name):
            assert t is None, name
            continue
        # each figure is a mean over launches, rounded to whole bytes on its own
        assert t is not None and abs(t["bytes_per_launch"] - t["fetch"] - t["write"]) <= 2, name
        assert bench.traffic_of(name, 1, doc["workload"] + "_other") is None
