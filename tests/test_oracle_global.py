"""Pins for the oracle's global tokens ([DistFlashAttn App. F]: global
attention, with the global tokens replicated on every worker), read as the
first G positions of the sequence on top of a local sliding window of W
tokens: a query at position p sees the keys at p - W + 1 .. p and every key
at a position below G that is not after p, each key once.

Each check is a fact the oracle does not compute itself: scalar loops over
explicitly listed keys, reductions to the window-only and plain causal
cases, torch's float64 attention with an explicit mask, finite differences,
the merge of two simpler masks, and an exhaustive check that the schedule
covers every visible (query, key) pair exactly once.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_bwd, attention_fwd, global_window_schedule, lse_merge,
                    window_schedule)
from oracle.schedule import GLOBAL

RNG = np.random.default_rng(23)


def brute_global(q, k, v, scale, q0, k0, win, g):
    """Scalar loops: the visible keys of (b, h, i) are listed by position."""
    b_, lq, hq, d = q.shape
    lk, hkv = k.shape[1], k.shape[2]
    grp = hq // hkv
    o = np.zeros((b_, lq, hq, d))
    lse = np.full((b_, hq, lq), -math.inf)
    for b in range(b_):
        for h in range(hq):
            gh = h // grp
            for i in range(lq):
                pos = q0 + i
                keys = [j for j in range(lk)
                        if k0 + j <= pos and (pos - (k0 + j) < win or k0 + j < g)]
                if not keys:
                    continue
                s = {j: scale * sum(q[b, i, h, t] * k[b, j, gh, t] for t in range(d)) for j in keys}
                m = max(s.values())
                lse[b, h, i] = m + math.log(sum(math.exp(s[j] - m) for j in keys))
                for j in keys:
                    w = math.exp(s[j] - lse[b, h, i])
                    for t in range(d):
                        o[b, i, h, t] += w * v[b, j, gh, t]
    return o, lse


CASES = [
    # (B, Lq, Lk, Hq, Hkv, d, q0, k0, W, G)
    (1, 9, 9, 1, 1, 3, 0, 0, 2, 3),    # diagonal: prefix of 3 globals, window 2
    (2, 5, 7, 2, 1, 2, 7, 0, 3, 2),    # off-diagonal pair: globals far behind the window
    (1, 6, 6, 4, 2, 3, 6, 0, 1, 6),    # every key of the first chunk global, W = 1
    (1, 6, 6, 2, 2, 2, 12, 6, 4, 3),   # keys past the global prefix: window only
    (1, 7, 7, 3, 3, 1, 0, 0, 1, 1),    # one global token (a sink) and each row itself
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    b, lq, lk, hq, hkv, d, q0, k0, win, g = case
    q = RNG.standard_normal((b, lq, hq, d))
    k = RNG.standard_normal((b, lk, hkv, d))
    v = RNG.standard_normal((b, lk, hkv, d))
    o, lse = attention_fwd(q, k, v, 0.7, True, q0, k0, window=win, n_global=g)
    ro, rl = brute_global(q, k, v, 0.7, q0, k0, win, g)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.max(np.abs(lse[fin] - rl[fin])) <= 1e-12
    assert np.max(np.abs(o - ro)) <= 1e-12


def test_reductions_to_window_only_and_to_causal():
    n, d = 20, 4
    q = RNG.standard_normal((1, n, 2, d))
    k = RNG.standard_normal((1, n, 2, d))
    v = RNG.standard_normal((1, n, 2, d))
    win_only = attention_fwd(q, k, v, 0.5, True, 0, 0, window=5)
    causal = attention_fwd(q, k, v, 0.5, True, 0, 0)
    # no global token: the window alone
    for x, y in zip(attention_fwd(q, k, v, 0.5, True, 0, 0, window=5, n_global=0), win_only):
        assert np.array_equal(x, y)
    # every position global, or a window covering the sequence: plain causal
    for w_, g in ((5, n), (n, 3), (n + 7, 1)):
        for x, y in zip(attention_fwd(q, k, v, 0.5, True, 0, 0, window=w_, n_global=g), causal):
            assert np.max(np.abs(x - y)) <= 1e-13


def test_torch_sdpa_with_explicit_mask():
    n, d, win, g = 40, 16, 6, 5
    q = RNG.standard_normal((1, n, 4, d))
    k = RNG.standard_normal((1, n, 4, d))
    v = RNG.standard_normal((1, n, 4, d))
    o, _ = attention_fwd(q, k, v, 1 / math.sqrt(d), True, 0, 0, window=win, n_global=g)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    mask = (j <= i) & ((i - j < win) | (j < g))
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    assert np.max(np.abs(o - ref.permute(0, 2, 1, 3).numpy())) <= 1e-12


def test_global_tokens_require_causal():
    x = np.zeros((1, 2, 1, 2))
    with pytest.raises(ValueError):
        attention_fwd(x, x, x, 1.0, False, n_global=1)


def test_two_masks_merge_to_the_combined_one():
    """Global keys (causal only) and the window over the remaining keys are
    disjoint key sets whose LSE merge is the combined mask."""
    n, d, win, g = 23, 3, 4, 6
    q = RNG.standard_normal((2, n, 2, d))
    k = RNG.standard_normal((2, n, 1, d))
    v = RNG.standard_normal((2, n, 1, d))
    o_ref, lse_ref = attention_fwd(q, k, v, 0.9, True, 0, 0, window=win, n_global=g)
    part_g = attention_fwd(q, k[:, :g], v[:, :g], 0.9, True, 0, 0)
    part_w = attention_fwd(q, k[:, g:], v[:, g:], 0.9, True, 0, g, window=win)
    o, lse = lse_merge([part_g[0], part_w[0]], [part_g[1], part_w[1]])
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


def _loss_and_grads(q, k, v, do, scale, win, g):
    o, lse = attention_fwd(q, k, v, scale, True, 0, 0, window=win, n_global=g)
    return float((o * do).sum()), attention_bwd(q, k, v, o, lse, do, scale, True, 0, 0,
                                                 window=win, n_global=g)


def test_backward_finite_differences():
    n, d, win, g, scale, h = 7, 2, 2, 2, 0.9, 1e-6
    q = RNG.standard_normal((1, n, 2, d))
    k = RNG.standard_normal((1, n, 1, d))
    v = RNG.standard_normal((1, n, 1, d))
    do = RNG.standard_normal((1, n, 2, d))
    _, (dq, dk, dv) = _loss_and_grads(q, k, v, do, scale, win, g)
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp, _ = _loss_and_grads(q, k, v, do, scale, win, g)
            arr[idx] = old - h
            lm, _ = _loss_and_grads(q, k, v, do, scale, win, g)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd))


def _item_keys(it, c, g):
    """Global positions of the keys an item of the global schedule covers."""
    kc = it[3]
    if kc == -1:
        return range(0, g)
    return range(max(kc * c, g if kc == 0 else 0), (kc + 1) * c)


def test_schedule_covers_every_visible_pair_exactly_once():
    for p in range(1, 8):
        for c in (1, 2, 3, 5):
            for win in range(1, p * c + 2):
                for g in range(1, c + 1):
                    items, steps = global_window_schedule(p, c, win, g)
                    assert (items, steps)[1] == window_schedule(p, c, win)[1]
                    assert items == sorted(items, key=lambda it: (it[0], it[1], it[3]))
                    assert [it for it in items if it[4] == GLOBAL] == \
                        [(0, w, w, -1, GLOBAL, w) for w in range(p)]
                    assert all(it[2] == it[1] == it[5] for it in items)  # no helpers
                    for pos in range(p * c):
                        a = pos // c
                        for j in range(pos + 1):
                            visible = pos - j < win or j < g
                            n_cover = sum(1 for it in items if it[2] == a and j in _item_keys(it, c, g))
                            # visible: exactly one item; hidden (j >= g then): at most one
                            # window item, whose window mask hides it
                            assert n_cover == 1 if visible else n_cover <= 1, (p, c, win, g, pos, j)
                    # every non-global item's key range is non-empty
                    assert all(len(_item_keys(it, c, g)) > 0 for it in items)


@pytest.mark.parametrize("p,c,win,g", [(3, 4, 3, 2), (4, 5, 7, 5), (5, 3, 2, 1), (2, 6, 13, 4)])
def test_chunked_schedule_then_merge_equals_monolithic(p, c, win, g):
    n, d = p * c, 3
    q = RNG.standard_normal((1, n, 2, d))
    k = RNG.standard_normal((1, n, 1, d))
    v = RNG.standard_normal((1, n, 1, d))
    o_ref, lse_ref = attention_fwd(q, k, v, 0.8, True, 0, 0, window=win, n_global=g)
    items, _ = global_window_schedule(p, c, win, g)
    parts = {}
    for it in items:
        a, kc = it[2], it[3]
        ks = list(_item_keys(it, c, g))
        k0, k1 = ks[0], ks[-1] + 1
        w_ = 0 if kc == -1 else win   # the global item: causal over the global keys only
        parts.setdefault(a, []).append(attention_fwd(
            q[:, a * c:(a + 1) * c], k[:, k0:k1], v[:, k0:k1], 0.8, True, a * c, k0, window=w_))
    for a in range(p):
        o, lse = lse_merge([x[0] for x in parts[a]], [x[1] for x in parts[a]])
        assert np.max(np.abs(o - o_ref[:, a * c:(a + 1) * c])) <= 1e-12
        assert np.max(np.abs(lse - lse_ref[:, :, a * c:(a + 1) * c])) <= 1e-12


def test_schedule_argument_checks():
    for g in (0, 6):
        with pytest.raises(ValueError):
            global_window_schedule(3, 5, 4, g)
