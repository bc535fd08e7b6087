"""dK/dV with the row split: pairs whose few key blocks see many query rows
(a short key range against a long query chunk, or the blocks a window band
reaches) run each block's steps as several workgroups and sum their
partials in a fixed order.  Checked against the float64 oracle, and two
runs must agree bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D
from long_context_exact_amd.synth import bf16_round

from _util import DEV, check_grad, rand, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("b,lq,lk,q0,k0,hq,hkv,dh,win", [
    (1, 8192, 256, 8192, 0, 2, 1, 128, 0),      # one key block, 512 steps: full pair
    (1, 4096, 300, 4000, 3800, 4, 2, 64, 0),    # ragged keys, causal edge inside the pair
    (1, 4096, 4096, 4096, 0, 2, 2, 128, 1000),  # window band: only the last keys see rows
    (2, 6144, 512, 6144, 0, 4, 4, 128, 0),      # batch 2
])
def test_split_dkdv_matches_oracle_and_repeats(b, lq, lk, q0, k0, hq, hkv, dh, win):
    print(f"case split {b} {lq} {lk} {q0} {k0} {hq} {hkv} {dh} {win}", flush=True)
    rng = np.random.default_rng(lq + 7 * lk + win)
    q = rand(rng, (b, lq, hq, dh), "bf16")
    k = rand(rng, (b, lk, hkv, dh), "bf16")
    v = rand(rng, (b, lk, hkv, dh), "bf16")
    d_o = rand(rng, (b, lq, hq, dh), "bf16")
    desc = D.make_desc(b, hq, hkv, dh, lq, lk, q0, k0, True, dh ** -0.5, "bf16", window=win)
    ro, rl = oracle.attention_fwd(q, k, v, dh ** -0.5, True, q0, k0, window=win)
    o_in = to_dev(bf16_round(ro.astype(np.float32)), "bf16")
    lse_in = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, d_o))
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, dh ** -0.5, True, q0, k0,
                                      window=win)
    runs = []
    for _ in range(2):
        delta = torch.empty_like(lse_in)
        dq = torch.zeros(b, lq, hq, dh, device=DEV)
        dk = torch.zeros(b, lk, hkv, dh, device=DEV)
        dv = torch.zeros(b, lk, hkv, dh, device=DEV)
        D.dfa_attn_bwd(desc, qd, kd, vd, o_in, lse_in, dod, delta, True, dq, dk, dv)
        torch.cuda.synchronize()
        runs.append((dq.clone(), dk.clone(), dv.clone()))
    for g, r, n in zip(runs[0], (rq, rk, rv), ("dQ", "dK", "dV")):
        check_grad(to_np(g), r, "bf16", n)
    for x, y in zip(*runs):
        assert torch.equal(x, y)
