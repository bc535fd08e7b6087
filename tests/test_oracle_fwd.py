"""Pins for the oracle's forward (exact causal softmax attention).

Each check is a fact the oracle does not compute itself: scalar Python
loops on tiny inputs, closed-form special cases, invariants of softmax, and
torch's float64 CPU attention where it defines the same quantity.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_fwd

RNG = np.random.default_rng(7)


def brute_force(q, k, v, scale, causal, q0, k0):
    """Scalar loops: for each (b, h, i) list the visible keys, take a plain
    two-pass softmax with math.exp / math.log and sum the weighted values."""
    b_, lq, hq, d = q.shape
    lk, hkv = k.shape[1], k.shape[2]
    grp = hq // hkv
    o = np.zeros((b_, lq, hq, d))
    lse = np.full((b_, hq, lq), -math.inf)
    for b in range(b_):
        for h in range(hq):
            g = h // grp
            for i in range(lq):
                keys = [j for j in range(lk) if (not causal) or (k0 + j <= q0 + i)]
                if not keys:
                    continue
                s = {j: scale * sum(q[b, i, h, t] * k[b, j, g, t] for t in range(d)) for j in keys}
                m = max(s.values())
                tot = sum(math.exp(s[j] - m) for j in keys)
                lse[b, h, i] = m + math.log(tot)
                for j in keys:
                    w = math.exp(s[j] - lse[b, h, i])
                    for t in range(d):
                        o[b, i, h, t] += w * v[b, j, g, t]
    return o, lse


CASES = [
    # (B, Lq, Lk, Hq, Hkv, d, causal, q0, k0)
    (1, 5, 5, 1, 1, 3, True, 0, 0),
    (2, 4, 6, 2, 1, 2, True, 3, 0),     # GQA, query chunk after key chunk start
    (1, 6, 3, 4, 2, 3, True, 2, 5),     # some rows see nothing
    (1, 3, 4, 3, 3, 1, False, 0, 0),    # non-causal, odd head count
    (1, 6, 6, 2, 2, 3, True, 6, 0),     # full (off-diagonal) chunk pair
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    b, lq, lk, hq, hkv, d, causal, q0, k0 = case
    q = RNG.standard_normal((b, lq, hq, d))
    k = RNG.standard_normal((b, lk, hkv, d))
    v = RNG.standard_normal((b, lk, hkv, d))
    scale = 0.7
    o, lse = attention_fwd(q, k, v, scale, causal, q0, k0)
    ob, lb = brute_force(q, k, v, scale, causal, q0, k0)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) <= 1e-13
    assert np.max(np.abs(o - ob)) <= 1e-13


def test_single_token_is_value():
    q = RNG.standard_normal((1, 1, 2, 4))
    k = RNG.standard_normal((1, 1, 2, 4))
    v = RNG.standard_normal((1, 1, 2, 4))
    o, lse = attention_fwd(q, k, v, 0.5)
    assert np.array_equal(o, v)
    for h in range(2):
        assert lse[0, h, 0] == pytest.approx(0.5 * float(q[0, 0, h] @ k[0, 0, h]), abs=1e-15)


def test_first_causal_row_is_v0():
    q = RNG.standard_normal((1, 40, 3, 8))
    k = RNG.standard_normal((1, 40, 3, 8))
    v = RNG.standard_normal((1, 40, 3, 8))
    o, _ = attention_fwd(q, k, v, 0.3)
    assert np.array_equal(o[0, 0], v[0, 0])


def test_zero_query_is_prefix_mean():
    """Q = 0 makes every visible score 0: O_i is the mean of V_0..V_i and
    LSE_i = ln(i + 1)."""
    n, h, d = 33, 2, 5
    q = np.zeros((1, n, h, d))
    k = RNG.standard_normal((1, n, h, d))
    v = RNG.standard_normal((1, n, h, d))
    o, lse = attention_fwd(q, k, v, 1.0)
    mean = np.cumsum(v[0], axis=0) / np.arange(1, n + 1)[:, None, None]
    assert np.max(np.abs(o[0] - mean)) <= 1e-13
    assert np.max(np.abs(lse[0] - np.log(np.arange(1, n + 1))[None, :])) <= 1e-13


def test_zero_scale_is_prefix_mean():
    n = 17
    q = RNG.standard_normal((1, n, 1, 4))
    k = RNG.standard_normal((1, n, 1, 4))
    v = RNG.standard_normal((1, n, 1, 4))
    o, _ = attention_fwd(q, k, v, 0.0)
    mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(o[0, :, 0] - mean)) <= 1e-13


def test_constant_value_gives_constant_output():
    q = RNG.standard_normal((1, 50, 2, 6)) * 3
    k = RNG.standard_normal((1, 50, 2, 6)) * 3
    v = np.broadcast_to(RNG.standard_normal((1, 1, 2, 6)), (1, 50, 2, 6)).copy()
    o, _ = attention_fwd(q, k, v, 0.4)
    assert np.max(np.abs(o - v)) <= 1e-13


def test_softmax_rows_sum_to_one():
    """exp(s_ij - LSE_i) over visible keys sums to one for every row, with the
    scores formed here by einsum from the raw inputs."""
    b, lq, lk, h, d = 2, 20, 30, 3, 7
    q0, k0 = 25, 10
    q = RNG.standard_normal((b, lq, h, d))
    k = RNG.standard_normal((b, lk, h, d))
    v = RNG.standard_normal((b, lk, h, d))
    _, lse = attention_fwd(q, k, v, 0.6, True, q0, k0)
    s = 0.6 * np.einsum("bihd,bjhd->bhij", q, k)
    vis = (k0 + np.arange(lk))[None, :] <= (q0 + np.arange(lq))[:, None]
    tot = np.where(vis[None, None], np.exp(s - lse[..., None]), 0.0).sum(-1)
    assert np.max(np.abs(tot - 1.0)) <= 1e-12


def test_key_shift_invariance():
    """Adding u to every key leaves O unchanged and moves LSE_i by
    sigma * <q_i, u>."""
    b, n, h, d = 1, 24, 2, 6
    q = RNG.standard_normal((b, n, h, d))
    k = RNG.standard_normal((b, n, h, d))
    v = RNG.standard_normal((b, n, h, d))
    u = RNG.standard_normal((1, 1, h, d))
    o1, l1 = attention_fwd(q, k, v, 0.5)
    o2, l2 = attention_fwd(q, k + u, v, 0.5)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    shift = 0.5 * np.einsum("bihd,bjhd->bhi", q, u)
    assert np.max(np.abs(l2 - l1 - shift)) <= 1e-12


def test_gqa_equals_repeated_heads():
    """Contiguous query-head groups: query head h reads key/value head h // G,
    which is multi-head attention on K, V repeated G times per head."""
    b, n, hq, hkv, d = 1, 19, 6, 2, 4
    q = RNG.standard_normal((b, n, hq, d))
    k = RNG.standard_normal((b, n, hkv, d))
    v = RNG.standard_normal((b, n, hkv, d))
    o1, l1 = attention_fwd(q, k, v, 0.5)
    o2, l2 = attention_fwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.5)
    assert np.max(np.abs(o1 - o2)) <= 1e-14
    assert np.max(np.abs(l1 - l2)) <= 1e-14


def test_matches_torch_sdpa_float64():
    """Library special case: torch's float64 CPU scaled-dot-product attention
    with the causal flag (queries and keys aligned at position 0)."""
    b, n, h, d = 2, 37, 3, 16
    q = RNG.standard_normal((b, n, h, d))
    k = RNG.standard_normal((b, n, h, d))
    v = RNG.standard_normal((b, n, h, d))
    o, lse = attention_fwd(q, k, v, 1 / 4)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1 / 4)
    assert np.max(np.abs(o - ref.permute(0, 2, 1, 3).numpy())) <= 1e-12
    s = (tq @ tk.transpose(-1, -2)) / 4
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(s.masked_fill(~mask, -torch.inf), dim=-1)
    assert np.max(np.abs(lse - ref_lse.numpy())) <= 1e-12


def test_empty_rows_are_zero_not_nan():
    q = RNG.standard_normal((1, 4, 1, 3))
    k = RNG.standard_normal((1, 4, 1, 3))
    v = RNG.standard_normal((1, 4, 1, 3))
    o, lse = attention_fwd(q, k, v, 1.0, True, 0, 10)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = attention_fwd(q[:, :0], k, v, 1.0)
    assert o.shape == (1, 0, 1, 3) and lse.shape == (1, 1, 0)


def test_peaky_scores_stay_finite():
    q = RNG.standard_normal((1, 64, 1, 8)) * 40
    k = RNG.standard_normal((1, 64, 1, 8)) * 40
    v = RNG.standard_normal((1, 64, 1, 8))
    o, lse = attention_fwd(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ob, lb = brute_force(q[:, :12], k[:, :12], v[:, :12], 1.0, True, 0, 0)
    assert np.max(np.abs(o[:, :12] - ob)) <= 1e-12
