"""GPU parity of the local sliding window ([DistFlashAttn App. F]) against the
float64 oracle: whole windowed sequences run through the window schedule,
merge and backward; single uneven pairs (including rows that see nothing);
the tile-visit map; and the window-free special case."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D
from long_context_exact_amd.runner import ChunkedCausalAttention

from _util import (DEV, case_seed, check_grad, check_lse, check_o, rand, run_sequence, to_dev,
                   to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare(att, q, k, v, d_o, got, dtype):
    c, win = att.chunk, att.window
    qf, kf, vf = (np.concatenate(x, axis=1).astype(np.float64) for x in (q, k, v))
    ro, rl = oracle.attention_fwd(qf, kf, vf, att.scale, True, 0, 0, window=win)
    for (a, cc), (op, lp) in got["partials"].items():
        po, pl = oracle.attention_fwd(q[a], k[cc], v[cc], att.scale, True, a * c, cc * c,
                                      window=win)
        check_o(op, po, dtype, f"O_part({a},{cc})")
        check_lse(lp, pl, dtype, f"LSE_part({a},{cc})")
    check_o(np.concatenate(got["o"], 1), ro, dtype, stored_bf16=dtype == "bf16")
    check_lse(np.concatenate(got["lse"], 2), rl, dtype)
    if d_o is not None:
        dof = np.concatenate(d_o, axis=1).astype(np.float64)
        rq, rk, rv = oracle.attention_bwd(qf, kf, vf, ro, rl, dof, att.scale, True, 0, 0,
                                          window=win)
        check_grad(np.concatenate(got["dq"], 1), rq, dtype, "dQ")
        check_grad(np.concatenate(got["dk"], 1), rk, dtype, "dK")
        check_grad(np.concatenate(got["dv"], 1), rv, dtype, "dV")


SEQ = [
    # (P, C, B, Hq, Hkv, D, window, dtype)
    (4, 200, 1, 4, 2, 128, 150, "bf16"),   # window inside a chunk, ragged tiles
    (3, 160, 1, 8, 1, 128, 160, "bf16"),   # window = chunk, GQA 8
    (4, 96, 1, 2, 2, 64, 250, "bf16"),     # window over two chunks: full + band pairs
    (3, 256, 1, 4, 1, 128, 1, "bf16"),     # each row sees only itself
    (2, 300, 2, 4, 4, 128, 33, "bf16"),    # narrow window, batch 2
    (5, 64, 1, 16, 2, 64, 100, "bf16"),    # GQA 8 at head_dim 64
    (3, 40, 1, 2, 1, 64, 50, "f32"),       # exact fp32 path
]


@pytest.mark.parametrize("case", SEQ)
def test_windowed_sequence_parity(case):
    P, C, B, Hq, Hkv, Dh, win, dt = case
    print(f"case window seq {case}", flush=True)
    rng = np.random.default_rng(case_seed(case))
    q = [rand(rng, (B, C, Hq, Dh), dt) for _ in range(P)]
    k = [rand(rng, (B, C, Hkv, Dh), dt) for _ in range(P)]
    v = [rand(rng, (B, C, Hkv, Dh), dt) for _ in range(P)]
    d_o = [rand(rng, (B, C, Hq, Dh), dt) for _ in range(P)]
    att = ChunkedCausalAttention(P, C, B, Hq, Hkv, Dh, dt, window=win)
    assert att.items == [tuple(x) for x in oracle.window_schedule(P, C, win)[0]]
    got = run_sequence(att, q, k, v, d_o)
    _compare(att, q, k, v, d_o, got, dt)


@pytest.mark.parametrize("lq,lk,q0,k0,win,dtype", [
    (100, 300, 1000, 800, 250, "bf16"),   # band: early rows see the key tail only
    (100, 300, 1200, 800, 250, "bf16"),   # some rows see nothing
    (257, 257, 0, 0, 100, "bf16"),        # diagonal with a window shorter than the chunk
    (64, 512, 512, 0, 448, "bf16"),       # band ending exactly at the chunk edge
    (100, 300, 1000, 800, 250, "f32"),
    (70, 70, 70, 0, 20, "f32"),
])
def test_windowed_pair(lq, lk, q0, k0, win, dtype):
    print(f"case window pair {lq} {lk} {q0} {k0} {win} {dtype}", flush=True)
    rng = np.random.default_rng(lq * 7919 + lk * 31 + win)
    hq, hkv, dh = 4, 2, 128
    q = rand(rng, (1, lq, hq, dh), dtype)
    k = rand(rng, (1, lk, hkv, dh), dtype)
    v = rand(rng, (1, lk, hkv, dh), dtype)
    desc = D.make_desc(1, hq, hkv, dh, lq, lk, q0, k0, True, dh ** -0.5, dtype, window=win)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o = torch.full((1, lq, hq, dh), 7.0, device=DEV)
    lse = torch.full((1, hq, lq), 7.0, device=DEV)
    D.dfa_attn_fwd_partial(desc, qd, kd, vd, o, lse)
    ro, rl = oracle.attention_fwd(q, k, v, dh ** -0.5, True, q0, k0, window=win)
    check_o(to_np(o), ro, dtype)
    check_lse(to_np(lse), rl, dtype)
    d_o = rand(rng, (1, lq, hq, dh), dtype)
    o_in = to_dev(ro.astype(np.float32), dtype)
    lse_in = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    delta = torch.empty_like(lse_in)
    dq = torch.zeros(1, lq, hq, dh, device=DEV)
    dk = torch.zeros(1, lk, hkv, dh, device=DEV)
    dv = torch.zeros(1, lk, hkv, dh, device=DEV)
    D.dfa_attn_bwd(desc, qd, kd, vd, o_in, lse_in, to_dev(d_o, dtype), delta, True, dq, dk, dv)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, dh ** -0.5, True, q0, k0,
                                      window=win)
    for g, r, n in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        if np.linalg.norm(r) == 0:
            assert np.all(to_np(g) == 0), n
        else:
            check_grad(to_np(g), r, dtype, n)


@pytest.mark.parametrize("lq,lk,q0,k0,hq,hkv,win", [
    (1000, 1000, 0, 0, 4, 4, 300), (1000, 1000, 1000, 0, 64, 8, 700),
    (300, 500, 4096, 3700, 4, 2, 500), (257, 257, 257, 257, 2, 2, 40), (96, 300, 200, 0, 4, 1, 150),
    # tile (10, 0) of 32 x 128 tiles: its closest pair is exactly `win` apart (skipped)
    (600, 600, 0, 0, 64, 8, 193),
])
def test_windowed_tile_visit_map_bit_exact(lq, lk, q0, k0, hq, hkv, win):
    print(f"case window tiles {lq} {lk} {q0} {k0} {hq} {hkv} {win}", flush=True)
    desc = D.make_desc(1, hq, hkv, 128, lq, lk, q0, k0, window=win)
    bm, bn = D.dfa_test_tile_shape(desc)
    q = torch.zeros(1, lq, hq, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, lk, hkv, 128, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(1, lq, hq, 128, device=DEV)
    lse = torch.empty(1, hq, lq, device=DEV)
    visits = torch.zeros(-(-lq // bm), -(-lk // bn), dtype=torch.uint8, device=DEV)
    D.dfa_test_fwd_tile_visits(desc, q, kv, kv, o, lse, visits)
    want = oracle.causal_tile_map(lq, lk, q0, k0, True, bm, bn, window=win)
    assert np.array_equal(visits.cpu().numpy(), want)


def test_window_covering_everything_is_bitwise_the_plain_path():
    rng = np.random.default_rng(5)
    lq = lk = 512
    hq, hkv, dh = 8, 2, 128
    q = rand(rng, (1, lq, hq, dh), "bf16")
    k = rand(rng, (1, lk, hkv, dh), "bf16")
    v = rand(rng, (1, lk, hkv, dh), "bf16")
    res = []
    for win in (0, 1 << 40):
        desc = D.make_desc(1, hq, hkv, dh, lq, lk, 512, 0, window=win)
        o = torch.empty(1, lq, hq, dh, device=DEV)
        lse = torch.empty(1, hq, lq, device=DEV)
        D.dfa_attn_fwd_partial(desc, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), o,
                               lse)
        torch.cuda.synchronize()
        res.append((to_np(o), to_np(lse)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
