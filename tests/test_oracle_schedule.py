"""Pins for the oracle's chunk-pair schedules and causal tile map against the
numbers the paper prints (golden/schedule_facts.json), a hand-typed P = 8
table of the adopted reading, exhaustive coverage checks for P = 1..32, and
an element-by-element enumeration of the tile map."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import balanced_schedule, causal_tile_map, unbalanced_schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FACTS = json.load(open(os.path.join(GOLDEN, "schedule_facts.json")))


def _grid(items, p, steps):
    g = [["-"] * p for _ in range(steps)]
    for step, w, a, c, kind, owner in items:
        assert g[step][w] == "-", "two items for one worker in one step"
        g[step][w] = f"{a},{c}" + ("*" if owner != w else "")
    return g


def test_p8_grid_matches_hand_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "schedule_p8_reading.txt"))
            if ln.strip() and not ln.startswith("#")]
    items, steps = balanced_schedule(8)
    assert _grid(items, 8, steps) == rows


def test_p4_grid():
    items, steps = balanced_schedule(4)
    assert _grid(items, 4, steps) == [["0,0", "1,1", "2,2", "3,3"],
                                      ["3,0*", "1,0", "2,1", "3,2"],
                                      ["-", "-", "2,0", "3,1"]]


@pytest.mark.parametrize("p", range(1, 33))
@pytest.mark.parametrize("balanced", [True, False])
def test_exhaustive_coverage(p, balanced):
    items, steps = (balanced_schedule if balanced else unbalanced_schedule)(p)
    pairs = [(a, c) for _, _, a, c, _, _ in items]
    assert sorted(pairs) == sorted((a, c) for a in range(p) for c in range(a + 1))
    assert len(set((s, w) for s, w, *_ in items)) == len(items)
    assert items == sorted(items, key=lambda it: (it[0], it[1]))
    assert steps == (1 + p // 2 if balanced else p)
    for step, w, a, c, kind, owner in items:
        assert owner == a and kind == (0 if a == c else 1)
        assert 0 <= step < steps and 0 <= w < p
        if owner != w:
            assert c == w, "a helper always uses its own key/value chunk"
        if not balanced:
            assert owner == w


def test_theoretical_speedups_at_8_workers():
    """Diagonal pair = one unit: one device does P(P+1)/2 units; P workers
    need `steps` time units."""
    f = FACTS["theoretical_speedup_over_one_device_p8"]
    for fn, want in ((balanced_schedule, f["balanced"]), (unbalanced_schedule, f["unbalanced"])):
        items, steps = fn(8)
        assert Fraction(len(items), steps) == Fraction(want).limit_denominator(10)


@pytest.mark.parametrize("p", range(1, 33))
def test_idle_fractions(p):
    items, steps = balanced_schedule(p)
    idle = Fraction(steps * p - len(items), steps * p)
    assert idle == (Fraction(1, p + 2) if p % 2 == 0 else 0)
    items, steps = unbalanced_schedule(p)
    assert Fraction(steps * p - len(items), steps * p) == Fraction(p - 1, 2 * p)


def test_idle_limits_and_gain():
    big = 4096
    b_items, b_steps = len(balanced_schedule(big)[0]), 1 + big // 2
    u_steps = big
    lim = FACTS["idle_fraction_limit"]
    assert abs((b_steps * big - b_items) / (b_steps * big) - lim["balanced_even_workers"]) < 1e-3
    assert abs((u_steps * big - b_items) / (u_steps * big) - lim["unbalanced"]) < 1e-3
    assert abs(u_steps / b_steps - FACTS["balancing_gain_limit"]["value"]) < 1e-3
    for p in (2, 4, 8, 16):
        assert Fraction(p, 1 + p // 2) == Fraction(2 * p, p + 2)


@pytest.mark.parametrize("p", [2, 4, 8, 16, 32])
def test_forward_traffic_per_worker_is_nd(p):
    """Per step after the first a worker either receives one K and one V chunk
    (owner) or receives a query chunk and returns an output chunk (helper):
    2 * C * d elements.  The busiest worker moves N * d = P * C * d."""
    items, _ = balanced_schedule(p)
    moved = [0] * p
    for step, w, *_ in items:
        if step > 0:
            moved[w] += 2            # units of C * d
    assert max(moved) == p * FACTS["communication_volume_per_worker"]["forward_in_units_of_N_d"]


def _tile_map_by_elements(lq, lk, q0, k0, causal, bm, bn):
    vis = ((k0 + np.arange(lk))[None, :] <= (q0 + np.arange(lq))[:, None]) if causal \
        else np.ones((lq, lk), bool)
    nqt, nkt = -(-lq // bm), -(-lk // bn)
    out = np.zeros((nqt, nkt), np.uint8)
    for qt in range(nqt):
        for kt in range(nkt):
            blk = vis[qt * bm:(qt + 1) * bm, kt * bn:(kt + 1) * bn]
            if blk.any():
                out[qt, kt] = 1 if blk.all() else 2
    return out


@pytest.mark.parametrize("case", [
    (64, 64, 0, 0, True, 16, 16), (70, 50, 0, 0, True, 16, 32), (33, 90, 40, 7, True, 8, 16),
    (40, 40, 100, 0, True, 16, 16), (40, 40, 0, 100, True, 16, 16), (37, 23, 0, 0, False, 8, 8),
    (100, 100, 0, 0, True, 32, 64),
    # tiles whose last key is exactly their first query (visible whole, no mask)
    (64, 64, 15, 0, True, 16, 16), (48, 64, 31, 0, True, 16, 32),
])
def test_tile_map_matches_element_enumeration(case):
    assert np.array_equal(causal_tile_map(*case), _tile_map_by_elements(*case))


@pytest.mark.parametrize("c,t", [(4096, 128), (1024, 64), (32768, 128)])
def test_diagonal_tile_counts_closed_form(c, t):
    m = causal_tile_map(c, c, 0, 0, True, t, t)
    n = c // t
    assert int((m > 0).sum()) == n * (n + 1) // 2
    assert int((m == 2).sum()) == n
    full = causal_tile_map(c, c, c, 0, True, t, t)
    assert np.all(full == 1)
