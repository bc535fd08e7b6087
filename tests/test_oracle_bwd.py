"""Pins for the oracle's backward from the saved O and LSE: central finite
differences of the forward, gradient identities, additivity over chunk-pair
blocks, and torch's float64 autograd of its own attention."""

import numpy as np
import pytest
import torch

from oracle import attention_bwd, attention_delta, attention_fwd

RNG = np.random.default_rng(23)


def _loss(q, k, v, do, scale, q0, k0):
    o, _ = attention_fwd(q, k, v, scale, True, q0, k0)
    return float((o * do).sum())


FD_CASES = [
    # (B, Lq, Lk, Hq, Hkv, d, q0, k0)
    (1, 4, 4, 1, 1, 3, 0, 0),
    (1, 5, 4, 4, 2, 2, 2, 0),     # GQA, offsets
    (2, 3, 5, 2, 1, 3, 4, 1),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_finite_differences(case):
    b, lq, lk, hq, hkv, d, q0, k0 = case
    q = RNG.standard_normal((b, lq, hq, d))
    k = RNG.standard_normal((b, lk, hkv, d))
    v = RNG.standard_normal((b, lk, hkv, d))
    do = RNG.standard_normal((b, lq, hq, d))
    scale = 0.8
    o, lse = attention_fwd(q, k, v, scale, True, q0, k0)
    grads = attention_bwd(q, k, v, o, lse, do, scale, True, q0, k0)
    h = 1e-6
    for x, g in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, q0, k0)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, q0, k0)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(num), 1e-30)
        assert err <= 1e-6, err


def _problem(b=1, n=40, hq=4, hkv=2, d=6):
    q = RNG.standard_normal((b, n, hq, d))
    k = RNG.standard_normal((b, n, hkv, d))
    v = RNG.standard_normal((b, n, hkv, d))
    do = RNG.standard_normal((b, n, hq, d))
    return q, k, v, do


def test_dk_sums_to_zero_and_dv_sums_to_do():
    """sum_j dS_ij = 0 for every row (softmax Jacobian), so dK summed over
    keys vanishes; dV summed over keys is dO summed over rows and group."""
    q, k, v, do = _problem()
    o, lse = attention_fwd(q, k, v, 0.4)
    _, dk, dv = attention_bwd(q, k, v, o, lse, do, 0.4)
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-12
    want = do.reshape(1, 40, 2, 2, 6).sum(axis=(1, 3))
    assert np.max(np.abs(dv.sum(axis=1) - want)) <= 1e-12


def test_zero_upstream_gives_zero_gradients():
    q, k, v, do = _problem()
    o, lse = attention_fwd(q, k, v, 0.4)
    for g in attention_bwd(q, k, v, o, lse, np.zeros_like(do), 0.4):
        assert np.all(g == 0)


def test_blocks_add_up_to_monolithic():
    """Chunk-pair blocks with the *final* O and LSE add up to the
    whole-sequence gradient (what the owner accumulates across items)."""
    q, k, v, do = _problem(n=36)
    o, lse = attention_fwd(q, k, v, 0.4)
    ref = attention_bwd(q, k, v, o, lse, do, 0.4)
    c = 12
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a in range(3):
        for kc in range(a + 1):
            qs, ks = slice(a * c, (a + 1) * c), slice(kc * c, (kc + 1) * c)
            g = attention_bwd(q[:, qs], k[:, ks], v[:, ks], o[:, qs], lse[:, :, qs], do[:, qs],
                              0.4, True, a * c, kc * c)
            dq[:, qs] += g[0]
            dk[:, ks] += g[1]
            dv[:, ks] += g[2]
    for x, y in zip((dq, dk, dv), ref):
        assert np.max(np.abs(x - y)) <= 1e-12


def test_delta_is_rowwise_dot():
    o = RNG.standard_normal((2, 5, 3, 4))
    do = RNG.standard_normal((2, 5, 3, 4))
    d = attention_delta(o, do)
    for b in range(2):
        for h in range(3):
            for i in range(5):
                assert d[b, h, i] == pytest.approx(float(np.dot(o[b, i, h], do[b, i, h])), abs=1e-14)


def test_matches_torch_autograd_float64():
    b, n, hq, hkv, d = 1, 30, 4, 2, 8
    q, k, v, do = _problem(b, n, hq, hkv, d)
    o, lse = attention_fwd(q, k, v, 0.3)
    dq, dk, dv = attention_bwd(q, k, v, o, lse, do, 0.3)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kr = tk.repeat_interleave(2, dim=2)
    vr = tv.repeat_interleave(2, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", tq, kr) * 0.3
    s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), -torch.inf)
    to = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vr)
    (to * torch.from_numpy(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-12


def test_rows_without_keys_contribute_nothing():
    q, k, v, do = _problem(n=8)
    o, lse = attention_fwd(q, k, v, 0.5, True, 0, 100)
    for g in attention_bwd(q, k, v, o, lse, do, 0.5, True, 0, 100):
        assert np.all(g == 0) and np.all(np.isfinite(g))
