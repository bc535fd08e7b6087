"""Pins for the oracle's local sliding window ([DistFlashAttn App. F]).

A query at global position p sees the keys at positions p - W + 1 .. p.
Each check is a fact the oracle does not compute itself: scalar loops over
explicitly listed keys, reductions to the unwindowed oracle on an explicit
key slice, closed forms, finite differences, torch's float64 attention with
an explicit mask, and an exhaustive check of the schedule's coverage.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_bwd, attention_fwd, causal_tile_map, lse_merge,
                    window_schedule)
from oracle.schedule import BAND, DIAG, FULL

RNG = np.random.default_rng(11)


def brute_window(q, k, v, scale, q0, k0, win):
    """Scalar loops: the visible keys of (b, h, i) are listed by position."""
    b_, lq, hq, d = q.shape
    lk, hkv = k.shape[1], k.shape[2]
    grp = hq // hkv
    o = np.zeros((b_, lq, hq, d))
    lse = np.full((b_, hq, lq), -math.inf)
    for b in range(b_):
        for h in range(hq):
            g = h // grp
            for i in range(lq):
                pos = q0 + i
                keys = [j for j in range(lk) if pos - win < k0 + j <= pos]
                if not keys:
                    continue
                s = {j: scale * sum(q[b, i, h, t] * k[b, j, g, t] for t in range(d)) for j in keys}
                m = max(s.values())
                lse[b, h, i] = m + math.log(sum(math.exp(s[j] - m) for j in keys))
                for j in keys:
                    w = math.exp(s[j] - lse[b, h, i])
                    for t in range(d):
                        o[b, i, h, t] += w * v[b, j, g, t]
    return o, lse


CASES = [
    # (B, Lq, Lk, Hq, Hkv, d, q0, k0, W)
    (1, 7, 7, 1, 1, 3, 0, 0, 3),
    (2, 5, 6, 2, 1, 2, 6, 0, 4),     # off-diagonal pair cut by the window
    (1, 6, 6, 4, 2, 3, 6, 0, 2),     # W = 2: only the nearest earlier token
    (1, 6, 6, 2, 2, 2, 12, 0, 5),    # every key too far: rows see nothing
    (1, 5, 5, 3, 3, 1, 0, 0, 1),     # W = 1: each row sees itself
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    b, lq, lk, hq, hkv, d, q0, k0, win = case
    q = RNG.standard_normal((b, lq, hq, d))
    k = RNG.standard_normal((b, lk, hkv, d))
    v = RNG.standard_normal((b, lk, hkv, d))
    o, lse = attention_fwd(q, k, v, 0.7, True, q0, k0, window=win)
    ro, rl = brute_window(q, k, v, 0.7, q0, k0, win)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.max(np.abs(lse[fin] - rl[fin]), initial=0.0) <= 1e-13
    assert np.max(np.abs(o - ro)) <= 1e-13


def test_row_equals_unwindowed_oracle_on_key_slice():
    """Row i of the windowed result is the plain (non-causal) attention of
    that one query over the explicit slice of its W keys."""
    lq, d, win = 40, 8, 9
    q = RNG.standard_normal((1, lq, 2, d))
    k = RNG.standard_normal((1, lq, 1, d))
    v = RNG.standard_normal((1, lq, 1, d))
    o, lse = attention_fwd(q, k, v, 0.3, True, 0, 0, window=win)
    for i in range(lq):
        lo = max(0, i - win + 1)
        ro, rl = attention_fwd(q[:, i:i + 1], k[:, lo:i + 1], v[:, lo:i + 1], 0.3, False)
        assert np.max(np.abs(o[:, i] - ro[:, 0])) <= 1e-13
        assert np.max(np.abs(lse[:, :, i] - rl[:, :, 0])) <= 1e-13


def test_window_one_is_identity_and_wide_window_is_causal():
    lq, d = 12, 4
    q = RNG.standard_normal((1, lq, 2, d))
    k = RNG.standard_normal((1, lq, 2, d))
    v = RNG.standard_normal((1, lq, 2, d))
    o, lse = attention_fwd(q, k, v, 0.5, True, 0, 0, window=1)
    assert np.max(np.abs(o - v)) <= 1e-15
    ref = 0.5 * np.einsum("bihd,bihd->bhi", q, k)
    assert np.max(np.abs(lse - ref)) <= 1e-14
    for win in (lq, lq + 5):
        ow, lw = attention_fwd(q, k, v, 0.5, True, 0, 0, window=win)
        oc, lc = attention_fwd(q, k, v, 0.5, True, 0, 0)
        assert np.array_equal(ow, oc) and np.array_equal(lw, lc)


def test_torch_sdpa_with_explicit_band_mask():
    lq, d, win = 33, 16, 10
    q = RNG.standard_normal((1, lq, 4, d))
    k = RNG.standard_normal((1, lq, 4, d))
    v = RNG.standard_normal((1, lq, 4, d))
    o, _ = attention_fwd(q, k, v, 1 / math.sqrt(d), True, 0, 0, window=win)
    i = torch.arange(lq)[:, None]
    j = torch.arange(lq)[None, :]
    mask = (j <= i) & (i - j < win)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    assert np.max(np.abs(o - ref.permute(0, 2, 1, 3).numpy())) <= 1e-12


def test_window_requires_causal():
    x = np.zeros((1, 2, 1, 2))
    with pytest.raises(ValueError):
        attention_fwd(x, x, x, 1.0, False, window=3)


@pytest.mark.parametrize("p,c,win", [(2, 5, 3), (3, 4, 4), (4, 3, 7), (4, 6, 13), (3, 5, 1)])
def test_chunked_window_schedule_then_merge_equals_monolithic(p, c, win):
    n, d = p * c, 3
    q = RNG.standard_normal((1, n, 2, d))
    k = RNG.standard_normal((1, n, 1, d))
    v = RNG.standard_normal((1, n, 1, d))
    o_ref, lse_ref = attention_fwd(q, k, v, 0.8, True, 0, 0, window=win)
    items, _ = window_schedule(p, c, win)
    parts = {}
    for (_, _, a, kc, _, _) in items:
        parts.setdefault(a, []).append(attention_fwd(
            q[:, a * c:(a + 1) * c], k[:, kc * c:(kc + 1) * c], v[:, kc * c:(kc + 1) * c],
            0.8, True, a * c, kc * c, window=win))
    for a in range(p):
        o, lse = lse_merge([x[0] for x in parts[a]], [x[1] for x in parts[a]])
        assert np.max(np.abs(o - o_ref[:, a * c:(a + 1) * c])) <= 1e-12
        assert np.max(np.abs(lse - lse_ref[:, :, a * c:(a + 1) * c])) <= 1e-12


def _loss_and_grads(q, k, v, do, scale, win):
    o, lse = attention_fwd(q, k, v, scale, True, 0, 0, window=win)
    return float((o * do).sum()), attention_bwd(q, k, v, o, lse, do, scale, True, 0, 0,
                                                 window=win)


def test_backward_finite_differences():
    n, d, win, scale, h = 6, 3, 3, 0.9, 1e-6
    q = RNG.standard_normal((1, n, 2, d))
    k = RNG.standard_normal((1, n, 1, d))
    v = RNG.standard_normal((1, n, 1, d))
    do = RNG.standard_normal((1, n, 2, d))
    _, (dq, dk, dv) = _loss_and_grads(q, k, v, do, scale, win)
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp, _ = _loss_and_grads(q, k, v, do, scale, win)
            arr[idx] = old - h
            lm, _ = _loss_and_grads(q, k, v, do, scale, win)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd))


def test_backward_identities_and_item_sum():
    p, c, win, d = 4, 5, 7, 4
    n = p * c
    q = RNG.standard_normal((1, n, 2, d))
    k = RNG.standard_normal((1, n, 1, d))
    v = RNG.standard_normal((1, n, 1, d))
    do = RNG.standard_normal((1, n, 2, d))
    o, lse = attention_fwd(q, k, v, 0.6, True, 0, 0, window=win)
    dq, dk, dv = attention_bwd(q, k, v, o, lse, do, 0.6, True, 0, 0, window=win)
    # every row sees itself, so its P sums to one: sum_j dS_ij = 0
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-12
    assert np.max(np.abs(dv.sum(axis=1)[:, 0] - do.sum(axis=(1, 2)))) <= 1e-12
    sq, sk, sv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for (_, _, a, kc, _, _) in window_schedule(p, c, win)[0]:
        rq, rk = slice(a * c, (a + 1) * c), slice(kc * c, (kc + 1) * c)
        gq, gk, gv = attention_bwd(q[:, rq], k[:, rk], v[:, rk], o[:, rq], lse[:, :, rq],
                                   do[:, rq], 0.6, True, a * c, kc * c, window=win)
        sq[:, rq] += gq
        sk[:, rk] += gk
        sv[:, rk] += gv
    for a_, b_ in ((sq, dq), (sk, dk), (sv, dv)):
        assert np.max(np.abs(a_ - b_)) <= 1e-12


def test_schedule_covers_exactly_the_visible_pairs():
    for p in range(1, 10):
        for c in (1, 2, 3, 5, 8):
            for win in range(1, p * c + 3):
                items, steps = window_schedule(p, c, win)
                got = {(it[2], it[3]) for it in items}
                assert len(got) == len(items)
                want = set()
                for a in range(p):
                    for kc in range(a + 1):
                        if any(0 <= i - j < win for i in range(a * c, (a + 1) * c)
                               for j in range(kc * c, (kc + 1) * c)):
                            want.add((a, kc))
                assert got == want, (p, c, win)
                assert steps == 1 + max(it[0] for it in items)
                assert all(it[2] == it[1] == it[5] for it in items)  # no helpers
                assert items == sorted(items, key=lambda it: (it[0], it[1]))
                for (t, w, a, kc, kind, _) in items:
                    dists = [i - j for i in range(a * c, (a + 1) * c)
                             for j in range(kc * c, (kc + 1) * c)]
                    if t == 0:
                        assert kind == DIAG
                    else:
                        assert kind == (FULL if max(dists) < win else BAND)


def test_schedule_worker_7_of_8_visits_chunks_6_and_7():
    """App. F: with a window no wider than a chunk, worker 7 loops over
    workers 6 and 7 only."""
    for c, win in ((1024, 1024), (1024, 2), (4096, 100)):
        items, steps = window_schedule(8, c, win)
        assert sorted(it[3] for it in items if it[1] == 7) == [6, 7]
        assert steps == 2


def test_tile_map_matches_element_enumeration():
    # the last case has tiles whose closest pair is exactly `win` apart (not visited)
    for (lq, lk, q0, k0, bm, bn, win) in [(64, 64, 0, 0, 16, 8, 20), (40, 48, 48, 0, 8, 16, 30),
                                          (32, 32, 64, 0, 8, 8, 40), (33, 47, 50, 3, 8, 16, 11),
                                          (64, 64, 0, 0, 16, 8, 25)]:
        m = causal_tile_map(lq, lk, q0, k0, True, bm, bn, window=win)
        for qt in range(m.shape[0]):
            for kt in range(m.shape[1]):
                rows = range(qt * bm, min((qt + 1) * bm, lq))
                cols = range(kt * bn, min((kt + 1) * bn, lk))
                vis = [0 <= (q0 + i) - (k0 + j) < win for i in rows for j in cols]
                want = 0 if not any(vis) else (1 if all(vis) else 2)
                assert m[qt, kt] == want, (qt, kt)
