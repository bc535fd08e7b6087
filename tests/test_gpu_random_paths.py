"""Seeded random chunk pairs of medium size (up to 2100 x 2100 tokens), drawn
so that the bf16 kernels take every launch path: fully visible pairs (the
mask-free kernels), masked pairs, diagonal pairs whose dK/dV runs as two row
bands (with a window shorter than the chunk, the first pairs each key block's
own rows with its window-edge rows), and pairs whose dK/dV rows are split
over workgroups with a fixed-order reduction.  Each pair is diagonal, fully
visible, a band (query chunk starting inside the key chunk), random offsets
or non-causal; lengths are ragged or whole 256-token blocks; windows of 1 to
5000 tokens; 1 to 64 query heads, grouping 1 to 8, batch 1 to 3, head_dim 64
or 128.  Forward (O, LSE) and backward (dQ, dK, dV from the oracle's O and
LSE) against the float64 oracle.  Which path a case takes comes from the
library's own host-side plan (launch count and workspace size), checked on
the CPU."""

from collections import Counter

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D

from _util import DEV, check_grad, check_lse, check_o, rand, to_dev, to_np


def _draw(n, seed=2023):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dh = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        grp = int(rng.choice([1, 2, 4, 8]))
        b = int(rng.choice([1, 1, 2, 3]))

        def length():
            if rng.random() < 0.6:
                return int(256 * rng.integers(1, 9))
            return int(rng.integers(1, 2100))

        kind = str(rng.choice(["diag", "diag", "full", "band", "random", "noncausal"]))
        lq = length()
        lk = lq if kind == "diag" else length()
        causal = kind != "noncausal"
        if kind == "diag":
            q0 = k0 = int(rng.choice([0, 256, 4096, 70000]))
        elif kind == "full":
            k0 = int(rng.choice([0, 1000]))
            q0 = k0 + lk + int(rng.integers(0, 300))
        elif kind == "band":
            k0 = 0
            q0 = lk - int(rng.integers(0, lk + 1))
        else:
            k0, q0 = (int(x) for x in rng.integers(0, 3000, size=2))
        win = 0
        if causal and rng.random() < 0.45:
            win = int(rng.choice([1, 31, 200, 512, 544, 800, 1024, 1536, 2048, 5000]))
        if b * hkv * grp * lq * lk > 24e6:  # keeps the oracle to about a second per case
            continue
        out.append((len(out), kind, b, lq, lk, q0, k0, hkv * grp, hkv, dh, causal, win))
    return out


CASES = _draw(48)


def _desc(case):
    _, _, b, lq, lk, q0, k0, hq, hkv, dh, causal, win = case
    return D.make_desc(b, hq, hkv, dh, lq, lk, q0, k0, causal, dh ** -0.5, "bf16", window=win)


def _path(case):
    """The dK/dV launch path the library plans for the case (host only)."""
    _, _, _, lq, lk, q0, k0, _, _, _, causal, win = case
    d = _desc(case)
    if D.dfa_attn_workspace_size(d, D.DFA_OP_BWD) > 0:
        return "row split"
    if D.dfa_test_bwd_launches(d, 1) > 1:
        # with a window shorter than the chunk the own rows and the rows at the
        # window's edge share one paired launch
        return "paired row bands" if 0 < win < lq else "row bands"
    sees_all = (not causal or q0 >= k0 + lk - 1) and (win == 0 or q0 + lq - 1 - k0 < win)
    return "mask-free" if sees_all and lk % 256 == 0 else "masked"


def test_cases_take_every_launch_path(dfa_lib):
    """CPU: the drawn cases reach every path (so the GPU test below covers them)."""
    paths = Counter(_path(c) for c in CASES)
    assert set(paths) == {"row split", "row bands", "paired row bands", "mask-free", "masked"}, paths


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_random_pair_on_its_path(case, dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    i, kind, b, lq, lk, q0, k0, hq, hkv, dh, causal, win = case
    print(f"case {case} path {_path(case)}", flush=True)
    rng = np.random.default_rng(9000 + i)
    scale = dh ** -0.5
    d = _desc(case)
    q = rand(rng, (b, lq, hq, dh), "bf16")
    k = rand(rng, (b, lk, hkv, dh), "bf16")
    v = rand(rng, (b, lk, hkv, dh), "bf16")
    d_o = rand(rng, (b, lq, hq, dh), "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = torch.full((b, lq, hq, dh), 7.0, device=DEV)
    lse = torch.full((b, hq, lq), 7.0, device=DEV)
    D.dfa_attn_fwd_partial(d, qd, kd, vd, o, lse)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, q0, k0, window=win)
    torch.cuda.synchronize()
    check_o(to_np(o), ro, "bf16", "O")
    check_lse(to_np(lse), rl, "bf16", "LSE")
    o_in = to_dev(ro.astype(np.float32), "bf16")
    lse_in = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, scale, causal, q0, k0,
                                      window=win)
    delta = torch.empty_like(lse_in)
    dq = torch.zeros(b, lq, hq, dh, device=DEV)
    dk = torch.zeros(b, lk, hkv, dh, device=DEV)
    dv = torch.zeros(b, lk, hkv, dh, device=DEV)
    D.dfa_attn_bwd(d, qd, kd, vd, o_in, lse_in, to_dev(d_o, "bf16"), delta, True, dq, dk, dv)
    torch.cuda.synchronize()
    for g, r, n in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        g = to_np(g)
        if np.linalg.norm(r) == 0:  # exactly zero in exact arithmetic: fp32 rounding level
            assert g.size == 0 or float(np.max(np.abs(g))) <= 1e-5, n
        else:
            check_grad(g, r, "bf16", n)
