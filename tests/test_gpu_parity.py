"""GPU parity of the HIP path (through the C ABI) against the float64 oracle,
element by element, at sizes the oracle finishes in seconds that still span
several tiles and a ragged tail; plus the special cases, the bit-exact tile
skipping map, determinism and the no-recompute backward."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D
from long_context_exact_amd.runner import ChunkedCausalAttention
from long_context_exact_amd.synth import WORKLOADS, bf16_round

from _util import (DEV, TD, case_seed, check_grad, check_lse, check_o, rand, run_sequence, to_dev,
                   to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_full(q, k, v, d_o, scale):
    qf, kf, vf = (np.concatenate(x, axis=1).astype(np.float64) for x in (q, k, v))
    o, lse = oracle.attention_fwd(qf, kf, vf, scale)
    res = {"o": o, "lse": lse}
    if d_o is not None:
        dof = np.concatenate(d_o, axis=1).astype(np.float64)
        res["dq"], res["dk"], res["dv"] = oracle.attention_bwd(qf, kf, vf, o, lse, dof, scale)
    return res


def _compare_sequence(att, q, k, v, d_o, got, dtype):
    c = att.chunk
    ref = _oracle_full(q, k, v, d_o, att.scale)
    for (a, cc), (op, lp) in got["partials"].items():
        ro, rl = oracle.attention_fwd(q[a], k[cc], v[cc], att.scale, True, a * c, cc * c)
        check_o(op, ro, dtype, f"O_part({a},{cc})")
        check_lse(lp, rl, dtype, f"LSE_part({a},{cc})")
    check_o(np.concatenate(got["o"], 1), ref["o"], dtype, stored_bf16=dtype == "bf16")
    check_lse(np.concatenate(got["lse"], 2), ref["lse"], dtype)
    if d_o is not None:
        check_grad(np.concatenate(got["dq"], 1), ref["dq"], dtype, "dQ")
        check_grad(np.concatenate(got["dk"], 1), ref["dk"], dtype, "dK")
        check_grad(np.concatenate(got["dv"], 1), ref["dv"], dtype, "dV")


def test_tiny_f32_workload():
    """Tiny fp32 workload, all 10 pairs + 4 merges + backward of all 10."""
    w = WORKLOADS["tiny_f32"]
    print(f"case tiny_f32 P={w.workers} C={w.chunk}", flush=True)
    q = [w.chunk_input(0, a) for a in range(w.workers)]
    k = [w.chunk_input(1, a) for a in range(w.workers)]
    v = [w.chunk_input(2, a) for a in range(w.workers)]
    d_o = [w.chunk_input(3, a) for a in range(w.workers)]
    att = ChunkedCausalAttention(w.workers, w.chunk, w.batch, w.heads_q, w.heads_kv, w.head_dim,
                                 "f32")
    assert len(att.items) == 10
    got = run_sequence(att, q, k, v, d_o)
    _compare_sequence(att, q, k, v, d_o, got, "f32")


SMALL = [
    # (P, C, B, Hq, Hkv, D, balanced)
    (3, 200, 2, 4, 2, 128, True),    # GQA 2, ragged tiles, batch 2
    (4, 96, 1, 3, 3, 64, True),      # irregular head count, head_dim 64
    (2, 256, 1, 8, 1, 128, True),    # GQA 8:1
    (5, 64, 1, 4, 1, 128, True),     # odd worker count, GQA 4
    (3, 130, 1, 2, 2, 128, False),   # unbalanced order, ragged
    (2, 160, 1, 16, 2, 64, True),    # GQA 8 at head_dim 64, two groups
]


@pytest.mark.parametrize("case", SMALL)
def test_bf16_sequence_parity(case):
    P, C, B, Hq, Hkv, Dh, bal = case
    print(f"case bf16 {case}", flush=True)
    rng = np.random.default_rng(case_seed(case))
    q = [rand(rng, (B, C, Hq, Dh), "bf16") for _ in range(P)]
    k = [rand(rng, (B, C, Hkv, Dh), "bf16") for _ in range(P)]
    v = [rand(rng, (B, C, Hkv, Dh), "bf16") for _ in range(P)]
    d_o = [rand(rng, (B, C, Hq, Dh), "bf16") for _ in range(P)]
    att = ChunkedCausalAttention(P, C, B, Hq, Hkv, Dh, "bf16", bal)
    got = run_sequence(att, q, k, v, d_o)
    _compare_sequence(att, q, k, v, d_o, got, "bf16")


def _fwd_pair(desc, q, k, v):
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = torch.full((desc.batch, desc.len_q, desc.heads_q, desc.head_dim), 7.0, device=DEV)
    lse = torch.full((desc.batch, desc.heads_q, desc.len_q), 7.0, device=DEV)
    D.dfa_attn_fwd_partial(desc, qd, kd, vd, o, lse)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


@pytest.mark.parametrize("lq,lk,q0,k0,causal,dtype", [
    (100, 37, 50, 80, True, "bf16"),    # first rows see nothing: O = 0, LSE = -inf
    (70, 129, 500, 0, True, "bf16"),    # full pair, ragged key tail
    (65, 65, 0, 0, False, "bf16"),      # non-causal
    (33, 300, 299, 0, True, "bf16"),    # query chunk inside a long key chunk
    (100, 37, 50, 80, True, "f32"),
    (40, 90, 0, 10, True, "f32"),
])
def test_uneven_pairs(lq, lk, q0, k0, causal, dtype):
    print(f"case pair {lq} {lk} {q0} {k0} {causal} {dtype}", flush=True)
    rng = np.random.default_rng(lq * 1000 + lk)
    hq, hkv, dh = 4, 2, 128
    q = rand(rng, (1, lq, hq, dh), dtype)
    k = rand(rng, (1, lk, hkv, dh), dtype)
    v = rand(rng, (1, lk, hkv, dh), dtype)
    desc = D.make_desc(1, hq, hkv, dh, lq, lk, q0, k0, causal, dh ** -0.5, dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o = torch.full((1, lq, hq, dh), 7.0, device=DEV)
    lse = torch.full((1, hq, lq), 7.0, device=DEV)
    D.dfa_attn_fwd_partial(desc, qd, kd, vd, o, lse)
    ro, rl = oracle.attention_fwd(q, k, v, dh ** -0.5, causal, q0, k0)
    check_o(to_np(o), ro, dtype)
    check_lse(to_np(lse), rl, dtype)
    # backward of the same pair with its own (O, LSE) as the "final" state
    d_o = rand(rng, (1, lq, hq, dh), dtype)
    o_in = to_dev(ro.astype(np.float32) if dtype == "f32" else bf16_round(ro.astype(np.float32)),
                  dtype)
    lse_in = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    delta = torch.empty_like(lse_in)
    dq = torch.zeros(1, lq, hq, dh, device=DEV)
    dk = torch.zeros(1, lk, hkv, dh, device=DEV)
    dv = torch.zeros(1, lk, hkv, dh, device=DEV)
    D.dfa_attn_bwd(desc, qd, kd, vd, o_in, lse_in, to_dev(d_o, dtype), delta, True, dq, dk, dv)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, dh ** -0.5, causal, q0, k0)
    for g, r, n in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        if np.linalg.norm(r) == 0:
            assert np.all(to_np(g) == 0), n
        else:
            check_grad(to_np(g), r, dtype, n)


def test_empty_key_chunk_fills_zero_and_neg_inf():
    desc = D.make_desc(1, 2, 2, 64, 50, 0)
    q = torch.zeros(1, 50, 2, 64, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    o = torch.full((1, 50, 2, 64), 3.0, device=DEV)
    lse = torch.full((1, 2, 50), 3.0, device=DEV)
    D.dfa_attn_fwd_partial(desc, q, kv, kv, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_first_causal_row_is_v0():
    rng = np.random.default_rng(5)
    c, hq, hkv, dh = 256, 8, 2, 128
    q, k, v = (rand(rng, s, "bf16") for s in ((1, c, hq, dh), (1, c, hkv, dh), (1, c, hkv, dh)))
    o, lse = _fwd_pair(D.make_desc(1, hq, hkv, dh, c, c), q, k, v)
    # Row 0 sees only key 0: its weight is exp2 of the rounding residual of
    # the one-FMA exponent argument (|residual| <= half an ulp of the scaled
    # max), so O_0 = V_0 to within 2 fp32 ulps rather than bit for bit.
    for h in range(hq):
        want = v[0, 0, h // 4].astype(np.float64)
        assert np.all(np.abs(o[0, 0, h] - want) <= 2.0 ** -22 * np.abs(want))
    # the same holds exactly on the fp32 path (plain exp of s - max = 0)
    q32, k32, v32 = (x.astype(np.float32) for x in (q, k, v))
    desc = D.make_desc(1, hq, hkv, dh, c, c, dtype="f32")
    o32 = torch.empty(1, c, hq, dh, device=DEV)
    l32 = torch.empty(1, hq, c, device=DEV)
    D.dfa_attn_fwd_partial(desc, to_dev(q32, "f32"), to_dev(k32, "f32"), to_dev(v32, "f32"),
                           o32, l32)
    for h in range(hq):
        assert np.array_equal(to_np(o32)[0, 0, h], v[0, 0, h // 4].astype(np.float64))


def test_special_cases_constant_v_zero_q_peaky():
    rng = np.random.default_rng(6)
    c, hq, dh = 300, 2, 128
    k = rand(rng, (1, c, hq, dh), "bf16")
    vconst = np.broadcast_to(rand(rng, (1, 1, hq, dh), "bf16"), (1, c, hq, dh)).copy()
    q = rand(rng, (1, c, hq, dh), "bf16")
    o, _ = _fwd_pair(D.make_desc(1, hq, hq, dh, c, c), q, k, vconst)
    assert np.max(np.abs(o - vconst)) <= 1e-2
    v = rand(rng, (1, c, hq, dh), "bf16")
    o, lse = _fwd_pair(D.make_desc(1, hq, hq, dh, c, c), np.zeros_like(q), k, v)
    mean = np.cumsum(v[0].astype(np.float64), axis=0) / np.arange(1, c + 1)[:, None, None]
    assert np.max(np.abs(o[0] - mean)) <= 1e-2
    assert np.max(np.abs(lse[0] - np.log(np.arange(1, c + 1))[None])) <= 1e-3 * np.log(c)
    qp = bf16_round((q * 8).astype(np.float32))
    o, lse = _fwd_pair(D.make_desc(1, hq, hq, dh, c, c), qp, k, v)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ro, rl = oracle.attention_fwd(qp, k, v, dh ** -0.5)
    check_o(o, ro, "bf16")
    check_lse(lse, rl, "bf16")


@pytest.mark.parametrize("lq,lk,q0,k0,hq,hkv", [
    (1000, 1000, 0, 0, 4, 4), (1000, 1000, 0, 0, 64, 8), (300, 500, 4096, 0, 4, 2),
    (257, 257, 257, 257, 2, 2), (96, 300, 200, 0, 4, 1),
    # a tile whose last key is exactly its first query (visited whole, unmasked):
    # 32 x 128 tiles (grouped heads) and 256 x 128 tiles (one head per kv head)
    (300, 400, 127, 0, 64, 8), (600, 700, 383, 0, 4, 4),
])
def test_tile_visit_map_bit_exact(lq, lk, q0, k0, hq, hkv):
    print(f"case tiles {lq} {lk} {q0} {k0} {hq} {hkv}", flush=True)
    desc = D.make_desc(1, hq, hkv, 128, lq, lk, q0, k0)
    bm, bn = D.dfa_test_tile_shape(desc)
    q = torch.zeros(1, lq, hq, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, lk, hkv, 128, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(1, lq, hq, 128, device=DEV)
    lse = torch.empty(1, hq, lq, device=DEV)
    visits = torch.zeros(-(-lq // bm), -(-lk // bn), dtype=torch.uint8, device=DEV)
    D.dfa_test_fwd_tile_visits(desc, q, kv, kv, o, lse, visits)
    want = oracle.causal_tile_map(lq, lk, q0, k0, True, bm, bn)
    assert np.array_equal(visits.cpu().numpy(), want)


def test_forward_and_backward_are_deterministic_and_remat_free():
    """Two forwards give bitwise-equal O and LSE; the backward from the saved
    state equals, bit for bit, a backward after recomputing the forward (the
    paper's checkpointing claim of no numerical difference)."""
    rng = np.random.default_rng(8)
    P, C, Hq, Hkv, Dh = 3, 192, 8, 2, 128
    att = ChunkedCausalAttention(P, C, 1, Hq, Hkv, Dh, "bf16")
    q = [rand(rng, att.q_shape(), "bf16") for _ in range(P)]
    k = [rand(rng, att.kv_shape(), "bf16") for _ in range(P)]
    v = [rand(rng, att.kv_shape(), "bf16") for _ in range(P)]
    d_o = [rand(rng, att.q_shape(), "bf16") for _ in range(P)]
    r1 = run_sequence(att, q, k, v, d_o)
    r2 = run_sequence(att, q, k, v, d_o)
    for key in ("o", "lse", "dq", "dk", "dv"):
        for a in range(P):
            assert np.array_equal(r1[key][a], r2[key][a]), key


# n below, at, and past multiples of the merge's eight partials per load group
@pytest.mark.parametrize("n,out", [(1, "f32"), (3, "bf16"), (8, "f32"), (9, "bf16"), (16, "f32"),
                                   (16, "bf16"), (17, "f32"), (64, "f32")])
def test_merge_parity(n, out):
    rng = np.random.default_rng(n)
    b, lq, h, dh = 2, 77, 3, 128
    os_ = [rng.standard_normal((b, lq, h, dh)).astype(np.float32) for _ in range(n)]
    ls_ = [(rng.standard_normal((b, h, lq)) * 20).astype(np.float32) for _ in range(n)]
    for r in range(n):                      # some empty partials, one all-empty row
        ls_[r][0, 0, r % lq] = -np.inf
        ls_[r][1, 2, 5] = -np.inf
    od = [torch.from_numpy(x).to(DEV) for x in os_]
    ld = [torch.from_numpy(x).to(DEV) for x in ls_]
    o = torch.empty(b, lq, h, dh, dtype=TD[out], device=DEV)
    lse = torch.empty(b, h, lq, device=DEV)
    D.dfa_lse_merge(od, ld, b, h, lq, dh, out, o, lse)
    ro, rl = oracle.lse_merge(os_, ls_)
    check_lse(to_np(lse), rl, "f32")
    # fp32 output: float32 arithmetic error only.  bf16 output: plus the final
    # round-to-nearest-even, half a bf16 ulp = 2^-9 relative (these synthetic
    # partials reach |O| ~ 4, where half an ulp is ~8e-3).
    err = np.abs(to_np(o) - ro)
    if out == "f32":
        assert err.max() <= 1e-5
    else:
        assert np.all(err <= 1e-5 + 2.0 ** -8 * np.abs(ro))
    if out == "f32":                        # in place over part 0
        D.dfa_lse_merge(od, ld, b, h, lq, dh, out, od[0], ld[0])
        assert np.max(np.abs(to_np(od[0]) - ro)) <= 1e-5
        check_lse(to_np(ld[0]), rl, "f32")


def test_backward_accumulates_into_existing_gradients():
    rng = np.random.default_rng(9)
    c, hq, hkv, dh = 128, 2, 2, 64
    q, k, v, d_o = (rand(rng, s, "bf16") for s in
                    ((1, c, hq, dh), (1, c, hkv, dh), (1, c, hkv, dh), (1, c, hq, dh)))
    desc = D.make_desc(1, hq, hkv, dh, c, c)
    ro, rl = oracle.attention_fwd(q, k, v, dh ** -0.5)
    o_in = to_dev(bf16_round(ro.astype(np.float32)), "bf16")
    lse = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    delta = torch.empty_like(lse)
    dq = torch.ones(1, c, hq, dh, device=DEV)
    dk = torch.ones(1, c, hkv, dh, device=DEV) * 2
    dv = torch.ones(1, c, hkv, dh, device=DEV) * 3
    D.dfa_attn_bwd(desc, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), o_in, lse,
                   to_dev(d_o, "bf16"), delta, True, dq, dk, dv)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, dh ** -0.5)
    check_grad(to_np(dq) - 1, rq, "bf16", "dQ")
    check_grad(to_np(dk) - 2, rk, "bf16", "dK")
    check_grad(to_np(dv) - 3, rv, "bf16", "dV")
    check_lse(to_np(delta), oracle.attention_delta(to_np(o_in), d_o), "f32", "delta")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_first_pair_still_writes_delta(dtype):
    """A query chunk whose first backward call has no keys (len_kv = 0) must
    still write delta when compute_delta is 1: the next pair, called with
    compute_delta = 0, reads it.  Compared with the oracle's gradient."""
    print(f"case empty first pair {dtype}", flush=True)
    rng = np.random.default_rng(case_seed(("empty-first", dtype)))
    hq, hkv, dh, lq, lk = 4, 2, 64, 96, 80
    q, d_o = (rand(rng, (1, lq, hq, dh), dtype) for _ in range(2))
    k, v = (rand(rng, (1, lk, hkv, dh), dtype) for _ in range(2))
    scale = dh ** -0.5
    ro, rl = oracle.attention_fwd(q, k, v, scale, True, 100, 0)
    o_in = to_dev(bf16_round(ro.astype(np.float32)) if dtype == "bf16" else
                  ro.astype(np.float32), dtype)
    lse = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    delta = torch.full_like(lse, float("nan"))
    dq = torch.zeros(1, lq, hq, dh, device=DEV)
    dk = torch.zeros(1, lk, hkv, dh, device=DEV)
    dv = torch.zeros_like(dk)
    empty = torch.zeros(1, 0, hkv, dh, device=DEV, dtype=TD[dtype])
    e32 = torch.zeros(1, 0, hkv, dh, device=DEV)
    D.dfa_attn_bwd(D.make_desc(1, hq, hkv, dh, lq, 0, 100, 0, dtype=dtype), to_dev(q, dtype),
                   empty, empty, o_in, lse, to_dev(d_o, dtype), delta, True, dq, e32, e32)
    D.dfa_attn_bwd(D.make_desc(1, hq, hkv, dh, lq, lk, 100, 0, dtype=dtype), to_dev(q, dtype),
                   to_dev(k, dtype), to_dev(v, dtype), None, lse, to_dev(d_o, dtype), delta, False,
                   dq, dk, dv)
    torch.cuda.synchronize()
    check_lse(to_np(delta), oracle.attention_delta(to_np(o_in), d_o), "f32", "delta")
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, scale, True, 100, 0)
    check_grad(to_np(dq), rq, dtype, "dQ")
    check_grad(to_np(dk), rk, dtype, "dK")
    check_grad(to_np(dv), rv, dtype, "dV")
