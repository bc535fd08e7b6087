"""GPU parity of the sliding window with replicated global tokens
([DistFlashAttn App. F]: global tokens replicated on every worker) against
the float64 oracle: whole sequences through the global-window schedule,
every partial, the merge and the backward."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd.runner import ChunkedCausalAttention

from _util import case_seed, check_grad, check_lse, check_o, rand, run_sequence

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _item_keys(kc, c, g):
    """Global key positions an item covers: the global prefix for kv chunk
    -1, chunk 0 past the prefix, or the whole chunk."""
    if kc == -1:
        return 0, g
    return (g if kc == 0 else kc * c), (kc + 1) * c


SEQ = [
    # (P, C, B, Hq, Hkv, D, window, n_global, dtype)
    (4, 200, 1, 4, 2, 128, 150, 16, "bf16"),   # window inside a chunk, ragged tiles
    (3, 160, 2, 8, 1, 128, 100, 64, "bf16"),   # batch 2: per-row calls for chunk-0 ranges
    (4, 96, 1, 2, 2, 64, 250, 96, "bf16"),     # every token of chunk 0 global
    (3, 256, 1, 4, 1, 128, 1, 1, "bf16"),      # one global token plus each row itself
    (5, 64, 2, 16, 2, 64, 33, 7, "bf16"),      # GQA 8 at head_dim 64, batch 2
    (3, 40, 1, 2, 1, 64, 50, 5, "f32"),        # exact fp32 path
    (2, 300, 2, 4, 4, 128, 20, 150, "f32"),    # fp32, batch 2, long global prefix
]


@pytest.mark.parametrize("case", SEQ)
def test_global_sequence_parity(case):
    P, C, B, Hq, Hkv, Dh, win, g, dt = case
    print(f"case global seq {case}", flush=True)
    rng = np.random.default_rng(case_seed(case))
    q = [rand(rng, (B, C, Hq, Dh), dt) for _ in range(P)]
    k = [rand(rng, (B, C, Hkv, Dh), dt) for _ in range(P)]
    v = [rand(rng, (B, C, Hkv, Dh), dt) for _ in range(P)]
    d_o = [rand(rng, (B, C, Hq, Dh), dt) for _ in range(P)]
    att = ChunkedCausalAttention(P, C, B, Hq, Hkv, Dh, dt, window=win, n_global=g)
    assert att.items == [tuple(x) for x in oracle.global_window_schedule(P, C, win, g)[0]]
    got = run_sequence(att, q, k, v, d_o)

    qf, kf, vf, dof = (np.concatenate(x, axis=1).astype(np.float64) for x in (q, k, v, d_o))
    for (a, kc), (op, lp) in got["partials"].items():
        k0, k1 = _item_keys(kc, C, g)
        po, pl = oracle.attention_fwd(q[a], kf[:, k0:k1], vf[:, k0:k1], att.scale, True, a * C,
                                      k0, window=0 if kc == -1 else win)
        check_o(op, po, dt, f"O_part({a},{kc})")
        check_lse(lp, pl, dt, f"LSE_part({a},{kc})")
    ro, rl = oracle.attention_fwd(qf, kf, vf, att.scale, True, 0, 0, window=win, n_global=g)
    check_o(np.concatenate(got["o"], 1), ro, dt, stored_bf16=dt == "bf16")
    check_lse(np.concatenate(got["lse"], 2), rl, dt)
    rq, rk, rv = oracle.attention_bwd(qf, kf, vf, ro, rl, dof, att.scale, True, 0, 0,
                                      window=win, n_global=g)
    check_grad(np.concatenate(got["dq"], 1), rq, dt, "dQ")
    check_grad(np.concatenate(got["dk"], 1), rk, dt, "dK")
    check_grad(np.concatenate(got["dv"], 1), rv, dt, "dV")
    # the global keys' gradient collects every worker's queries
    assert np.abs(np.concatenate(got["dv"], 1)[:, :g]).max() > 0


def test_global_tokens_need_a_window(dfa_lib):
    with pytest.raises(ValueError):
        ChunkedCausalAttention(2, 64, 1, 2, 2, 64, "bf16", window=0, n_global=4)
