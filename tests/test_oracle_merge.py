"""Pins for the oracle's LSE merge: chunked-then-merged equals the monolithic
exact attention, plus the algebraic identities of a log-sum-exp combine."""

import itertools
import math

import numpy as np
import pytest

from oracle import attention_fwd, lse_merge

RNG = np.random.default_rng(11)


def _chunked(q, k, v, scale, bounds):
    """Partials of the whole query range against each key chunk [a, b)."""
    parts = [attention_fwd(q, k[:, a:b], v[:, a:b], scale, True, 0, a) for a, b in bounds]
    return [p[0] for p in parts], [p[1] for p in parts]


@pytest.mark.parametrize("p", [1, 2, 3, 4, 8])
def test_chunked_merge_equals_monolithic(p):
    b, n, hq, hkv, d = 2, 48, 4, 2, 8
    q = RNG.standard_normal((b, n, hq, d))
    k = RNG.standard_normal((b, n, hkv, d))
    v = RNG.standard_normal((b, n, hkv, d))
    o_ref, l_ref = attention_fwd(q, k, v, 0.35)
    c = n // p
    bounds = [(i * c, n if i == p - 1 else (i + 1) * c) for i in range(p)]
    o, lse = lse_merge(*_chunked(q, k, v, 0.35, bounds))
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - l_ref)) <= 1e-12


def test_uneven_chunks_and_query_chunks():
    """Query chunks at their global offsets against uneven key chunks."""
    b, n, h, d = 1, 41, 2, 5
    q = RNG.standard_normal((b, n, h, d))
    k = RNG.standard_normal((b, n, h, d))
    v = RNG.standard_normal((b, n, h, d))
    o_ref, l_ref = attention_fwd(q, k, v, 0.5)
    cuts = [0, 7, 8, 20, 33, 41]
    for qa, qb in zip(cuts[:-1], cuts[1:]):
        parts = [attention_fwd(q[:, qa:qb], k[:, ka:kb], v[:, ka:kb], 0.5, True, qa, ka)
                 for ka, kb in zip(cuts[:-1], cuts[1:])]
        o, lse = lse_merge([x[0] for x in parts], [x[1] for x in parts])
        assert np.max(np.abs(o - o_ref[:, qa:qb])) <= 1e-12
        assert np.max(np.abs(lse - l_ref[:, :, qa:qb])) <= 1e-12


def test_single_part_is_identity():
    o = RNG.standard_normal((1, 5, 2, 3))
    lse = RNG.standard_normal((1, 2, 5))
    mo, ml = lse_merge([o], [lse])
    assert np.max(np.abs(mo - o)) <= 1e-15 and np.max(np.abs(ml - lse)) <= 1e-15


def test_empty_part_is_identity():
    o = RNG.standard_normal((1, 5, 2, 3))
    lse = RNG.standard_normal((1, 2, 5))
    mo, ml = lse_merge([o, np.zeros_like(o)], [lse, np.full_like(lse, -np.inf)])
    assert np.array_equal(mo, o) and np.array_equal(ml, lse)
    mo, ml = lse_merge([np.zeros_like(o)] * 2, [np.full_like(lse, -np.inf)] * 2)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))


def test_identical_parts_add_ln2():
    o = RNG.standard_normal((2, 6, 3, 4))
    lse = RNG.standard_normal((2, 3, 6)) * 5
    mo, ml = lse_merge([o, o], [lse, lse])
    assert np.max(np.abs(mo - o)) <= 1e-14
    assert np.max(np.abs(ml - lse - math.log(2))) <= 1e-13


def test_permutation_invariance():
    n = 4
    os_ = [RNG.standard_normal((1, 7, 2, 3)) for _ in range(n)]
    ls_ = [RNG.standard_normal((1, 2, 7)) * 4 for _ in range(n)]
    ref_o, ref_l = lse_merge(os_, ls_)
    for perm in itertools.permutations(range(n)):
        o, lse = lse_merge([os_[i] for i in perm], [ls_[i] for i in perm])
        assert np.max(np.abs(o - ref_o)) <= 1e-14
        assert np.max(np.abs(lse - ref_l)) <= 1e-14


def test_far_apart_lse_values():
    """A part 800 nats below the other contributes nothing and causes no
    overflow / NaN."""
    o1 = RNG.standard_normal((1, 3, 1, 2))
    o2 = RNG.standard_normal((1, 3, 1, 2))
    l1 = np.full((1, 1, 3), 400.0)
    l2 = np.full((1, 1, 3), -400.0)
    mo, ml = lse_merge([o1, o2], [l1, l2])
    assert np.max(np.abs(mo - o1)) <= 1e-15
    assert np.max(np.abs(ml - 400.0)) <= 1e-13


def test_rows_every_part_leaves_empty():
    """Rows whose every partial saw no key (LSE = -inf everywhere) merge to
    O = 0 and LSE = -inf; the other rows are merged as usual."""
    o1 = RNG.standard_normal((1, 4, 2, 3))
    o2 = RNG.standard_normal((1, 4, 2, 3))
    l1 = RNG.standard_normal((1, 2, 4))
    l2 = RNG.standard_normal((1, 2, 4))
    for lx in (l1, l2):
        lx[0, 1, 2] = -np.inf        # head 1, row 2: empty in every part
    o1[0, 2, 1] = 0.0
    o2[0, 2, 1] = 0.0
    mo, ml = lse_merge([o1, o2], [l1, l2])
    assert ml[0, 1, 2] == -np.inf and np.all(mo[0, 2, 1] == 0.0)
    assert np.all(np.isfinite(np.delete(ml.reshape(-1), 1 * 4 + 2)))
    # a live row: both parts weighted by their share of the union's mass
    lse = np.logaddexp(l1[0, 0, 0], l2[0, 0, 0])
    assert abs(ml[0, 0, 0] - lse) <= 1e-14
    want = np.exp(l1[0, 0, 0] - lse) * o1[0, 0, 0] + np.exp(l2[0, 0, 0] - lse) * o2[0, 0, 0]
    assert np.max(np.abs(mo[0, 0, 0] - want)) <= 1e-14
