"""Seeded random chunk pairs and whole sequences against the float64 oracle.

Pairs: head grouping 1..8,
head_dim 64 and 128, batch 1 or 2, query and key lengths from 1 to 400 with
arbitrary global offsets (so tiles are ragged and the causal edge or the
window band falls anywhere), causal or not, with and without a sliding
window, bf16 and fp32.  Forward (O, LSE) and backward (dQ, dK, dV from the
oracle's final O and LSE) of every pair.  Sequences: 1 to 6 workers of 1 to 160
tokens through the runner (balanced or unbalanced schedule, sliding window,
global tokens), every partial, the merge and the backward."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D
from long_context_exact_amd.synth import bf16_round

from _util import DEV, check_grad, check_lse, check_o, rand, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _draw(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8]))
        dh = int(rng.choice([64, 128]))
        b = int(rng.choice([1, 2]))
        lq, lk = (int(x) for x in rng.integers(1, 401, size=2))
        q0 = int(rng.integers(0, 601))
        k0 = max(0, q0 + int(rng.integers(-500, 101)))  # mostly keys at or before the queries
        causal = bool(rng.random() < 0.8)
        window = int(rng.integers(1, 301)) if causal and rng.random() < 0.4 else 0
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        cases.append((i, b, lq, lk, q0, k0, hkv * group, hkv, dh, causal, window, dtype))
    return cases


def _check_grad_or_zero(g, r, dt, n):
    """A gradient that is exactly zero in exact arithmetic (every row sees at
    most one key: P = 1, O = V, dS = P (dP - D) = 0) comes out of the kernels
    at fp32 rounding level (a few 1e-7), not bitwise zero: the bound there is
    the absolute 1e-5 of the exact path; anything else takes the usual check."""
    if np.linalg.norm(r) == 0:
        err = float(np.max(np.abs(g))) if g.size else 0.0
        assert err <= 1e-5, f"{n}: exact zero, got max |g| {err}"
    else:
        check_grad(g, r, dt, n)


def _draw_long(n, seed=79):
    """Long query chunks against short key chunks: few key blocks with many
    rows each, the shape for which dK/dV splits a block's rows over several
    workgroups."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8]))
        dh = int(rng.choice([64, 128]))
        b = int(rng.choice([1, 2]))
        lq, lk = int(rng.integers(1024, 4097)), int(rng.integers(1, 701))
        q0 = int(rng.integers(0, 3000))
        k0 = max(0, q0 + int(rng.integers(-2000, 50)))
        causal = bool(rng.random() < 0.85)
        window = int(rng.integers(1, 1500)) if causal and rng.random() < 0.4 else 0
        dtype = "f32" if rng.random() < 0.15 else "bf16"
        cases.append((100 + i, b, lq, lk, q0, k0, hkv * group, hkv, dh, causal, window, dtype))
    return cases


@pytest.mark.parametrize("case", _draw(48) + _draw_long(8), ids=lambda c: f"r{c[0]}")
def test_random_pair(case):
    i, b, lq, lk, q0, k0, hq, hkv, dh, causal, win, dt = case
    print(f"case random pair {case}", flush=True)
    rng = np.random.default_rng(1000 + i)
    scale = dh ** -0.5
    q = rand(rng, (b, lq, hq, dh), dt)
    k = rand(rng, (b, lk, hkv, dh), dt)
    v = rand(rng, (b, lk, hkv, dh), dt)
    d_o = rand(rng, (b, lq, hq, dh), dt)
    desc = D.make_desc(b, hq, hkv, dh, lq, lk, q0, k0, causal, scale, dt, window=win)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    o = torch.full((b, lq, hq, dh), 7.0, device=DEV)
    lse = torch.full((b, hq, lq), 7.0, device=DEV)
    D.dfa_attn_fwd_partial(desc, qd, kd, vd, o, lse)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, q0, k0, window=win)
    check_o(to_np(o), ro, dt)
    check_lse(to_np(lse), rl, dt)

    o_in = to_dev(ro.astype(np.float32) if dt == "f32" else bf16_round(ro.astype(np.float32)), dt)
    lse_in = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    delta = torch.empty_like(lse_in)
    dq = torch.zeros(b, lq, hq, dh, device=DEV)
    dk = torch.zeros(b, lk, hkv, dh, device=DEV)
    dv = torch.zeros(b, lk, hkv, dh, device=DEV)
    D.dfa_attn_bwd(desc, qd, kd, vd, o_in, lse_in, to_dev(d_o, dt), delta, True, dq, dk, dv)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, scale, causal, q0, k0,
                                      window=win)
    for g, r, n in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        _check_grad_or_zero(to_np(g), r, dt, n)


def _draw_sequences(n, seed=2025):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        p = int(rng.integers(1, 7))
        c = int(rng.integers(1, 161))
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        dh = int(rng.choice([64, 128]))
        b = int(rng.choice([1, 2]))
        dt = "f32" if rng.random() < 0.25 else "bf16"
        kind = rng.random()
        win = g = 0
        balanced = True
        if kind < 0.3:
            win = int(rng.integers(1, p * c + 2))
        elif kind < 0.5:
            win = int(rng.integers(1, p * c + 2))
            g = int(rng.integers(1, c + 1))
        elif kind < 0.6:
            balanced = False
        cases.append((i, p, c, b, hq, hkv, dh, dt, win, g, balanced))
    return cases


@pytest.mark.parametrize("case", _draw_sequences(24), ids=lambda c: f"s{c[0]}")
def test_random_sequence(case):
    """Whole sequences through the runner (schedule, every partial, the
    merge, the backward) against the oracle's whole-sequence attention."""
    from long_context_exact_amd.runner import ChunkedCausalAttention
    from _util import run_sequence
    i, p, c, b, hq, hkv, dh, dt, win, g, balanced = case
    print(f"case random sequence {case}", flush=True)
    rng = np.random.default_rng(2000 + i)
    q = [rand(rng, (b, c, hq, dh), dt) for _ in range(p)]
    k = [rand(rng, (b, c, hkv, dh), dt) for _ in range(p)]
    v = [rand(rng, (b, c, hkv, dh), dt) for _ in range(p)]
    d_o = [rand(rng, (b, c, hq, dh), dt) for _ in range(p)]
    att = ChunkedCausalAttention(p, c, b, hq, hkv, dh, dt, balanced=balanced, window=win,
                                 n_global=g)
    got = run_sequence(att, q, k, v, d_o)
    qf, kf, vf, dof = (np.concatenate(x, axis=1).astype(np.float64) for x in (q, k, v, d_o))
    ro, rl = oracle.attention_fwd(qf, kf, vf, att.scale, True, 0, 0, window=win, n_global=g)
    check_o(np.concatenate(got["o"], 1), ro, dt, stored_bf16=dt == "bf16")
    check_lse(np.concatenate(got["lse"], 2), rl, dt)
    rq, rk, rv = oracle.attention_bwd(qf, kf, vf, ro, rl, dof, att.scale, True, 0, 0,
                                      window=win, n_global=g)
    check_grad(np.concatenate(got["dq"], 1), rq, dt, "dQ")
    check_grad(np.concatenate(got["dk"], 1), rk, dt, "dK")
    check_grad(np.concatenate(got["dv"], 1), rv, dt, "dV")
