"""Element offsets past 2^31: one chunk pair whose key and value tensors hold
more than 2^31 elements (2^21 + 4099 keys x 8 heads x 128), so every kernel
of the pair (the V transpose, the forward, dK/dV, dQ, delta) addresses
elements whose index needs 64-bit arithmetic: every key at or after 2^21
sits past the 2^31-element mark of K and V and past the 2^32-byte mark of
the fp32 dK and dV.  The queries sit just after the keys' start of the last
tile (causal edge inside the last, ragged key block).  Checked against the
float64 oracle on the first and the last head (every query row; dK, dV on
keys at both ends of the key range, including all keys past the mark)."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D
from long_context_exact_amd.synth import bf16_bits, bf16_round

from _util import DEV, check_grad, check_lse, check_o, rand, rel_fro

pytestmark = pytest.mark.gpu

L = (1 << 21) + 4099   # keys: L * 8 * 128 > 2^31 elements
LQ = 40                # query rows: one full 32-row tile and a ragged one
H = 8                  # query heads = key/value heads (group 1: head h reads kv head h)
DH = 128
Q0 = L - 20            # rows 0..19 see keys up to L - 20 + i, rows 20.. see every key
HEADS = (0, H - 1)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _kv_bits(seed):
    """[L, H, DH] bf16 bits: one float32 draw of [L, DH] rounded to bf16, each
    head a different rotation of it along the key axis (distinct heads
    without drawing H times as many numbers)."""
    base = bf16_bits(bf16_round(
        np.random.default_rng(seed).standard_normal((L, DH), dtype=np.float32)))
    out = np.empty((L, H, DH), dtype=np.uint16)
    for h in range(H):  # head h: base rotated down by 997 * h keys
        s = 997 * h
        out[s:, h, :] = base[:L - s]
        out[:s, h, :] = base[L - s:]
    return out


def _head(bits, h):
    """float64 [1, L, 1, DH] of one head, from the same bits the GPU gets."""
    x = (bits[:, h, :].astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float64)[None, :, None, :]


def test_pair_past_2_31_elements():
    print(f"case large pair L={L} LQ={LQ} H={H} d={DH}", flush=True)
    kb, vb = _kv_bits(11), _kv_bits(12)
    rng = np.random.default_rng(13)
    q = rand(rng, (1, LQ, H, DH), "bf16")
    d_o = rand(rng, (1, LQ, H, DH), "bf16")
    scale = DH ** -0.5

    # oracle forward on the checked heads
    ref = {}
    for h in HEADS:
        kh, vh = _head(kb, h), _head(vb, h)
        ro, rl = oracle.attention_fwd(q[:, :, h:h + 1], kh, vh, scale, True, Q0, 0)
        ref[h] = (kh, vh, ro, rl)

    k_d = torch.from_numpy(kb).to(DEV).view(torch.bfloat16)[None]  # [1, L, H, DH]
    v_d = torch.from_numpy(vb).to(DEV).view(torch.bfloat16)[None]
    q_d = torch.from_numpy(q).to(DEV).to(torch.bfloat16)
    do_d = torch.from_numpy(d_o).to(DEV).to(torch.bfloat16)
    desc = D.make_desc(1, H, H, DH, LQ, L, Q0, 0, True, scale, "bf16")
    o_part = torch.empty(1, LQ, H, DH, device=DEV)
    lse = torch.empty(1, H, LQ, device=DEV)
    D.dfa_attn_fwd_partial(desc, q_d, k_d, v_d, o_part, lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o_part).all() and torch.isfinite(lse).all()
    for h in HEADS:
        _, _, ro, rl = ref[h]
        check_o(o_part[:, :, h:h + 1].cpu().numpy().astype(np.float64), ro, "bf16", f"O head {h}")
        check_lse(lse[:, h:h + 1].cpu().numpy().astype(np.float64), rl, "bf16", f"LSE head {h}")

    # backward from the saved output: the checked heads get the oracle's
    # O (delivered in bf16) and LSE; the other heads keep the forward's (with
    # one key/value head per query head they do not touch the checked ones)
    o_in = o_part.clone()
    lse_in = lse.clone()
    for h in HEADS:
        _, _, ro, rl = ref[h]
        o_in[:, :, h] = torch.from_numpy(bf16_round(ro[:, :, 0].astype(np.float32))).to(DEV)
        lse_in[:, h] = torch.from_numpy(rl[:, 0].astype(np.float32)).to(DEV)
    o_in = o_in.to(torch.bfloat16)
    delta = torch.empty(1, H, LQ, device=DEV)
    dq = torch.zeros(1, LQ, H, DH, device=DEV)
    dk = torch.zeros(1, L, H, DH, device=DEV)
    dv = torch.zeros(1, L, H, DH, device=DEV)
    D.dfa_attn_bwd(desc, q_d, k_d, v_d, o_in, lse_in, do_d, delta, True, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all()

    # The oracle backward from the final O and LSE is exact on any block of
    # (rows, keys): dQ over every key for rows R0..R0+7 (across the causal
    # edge at row 20), dK and dV over every row for two key ranges, the first
    # 300 keys and the last 4399 (past the 2^31-element mark from key 2^21 on,
    # the last 20 on the causal edge).
    # (The oracle's dQ is summed over key blocks of 2^18: the backward is
    # linear in the keys, and the blocks keep its temporaries small.)
    r0, r1 = 16, 24
    ranges = ((0, 300), (L - 4399, L))
    for h in HEADS:
        kh, vh, ro, rl = ref[h]
        qh, doh = q[:, :, h:h + 1], d_o[:, :, h:h + 1]
        o_h = o_in[:, :, h:h + 1].float().cpu().numpy().astype(np.float64)
        rq = 0.0
        for k0 in range(0, L, 1 << 18):
            k1 = min(L, k0 + (1 << 18))
            rq = rq + oracle.attention_bwd(qh[:, r0:r1], kh[:, k0:k1], vh[:, k0:k1],
                                           o_h[:, r0:r1], rl[:, :, r0:r1], doh[:, r0:r1],
                                           scale, True, Q0 + r0, k0)[0]
        check_grad(dq[:, r0:r1, h:h + 1].cpu().numpy().astype(np.float64), rq, "bf16",
                   f"dQ head {h}")
        for k0, k1 in ranges:
            _, rk, rv = oracle.attention_bwd(qh, kh[:, k0:k1], vh[:, k0:k1], o_h, rl, doh,
                                             scale, True, Q0, k0)
            gk = dk[0, k0:k1, h].cpu().numpy().astype(np.float64)
            gv = dv[0, k0:k1, h].cpu().numpy().astype(np.float64)
            assert np.all(np.isfinite(gk)) and np.all(np.isfinite(gv))
            assert rel_fro(gk, rk[0, :, 0]) <= 2e-2, f"dK head {h} keys {k0}..: {rel_fro(gk, rk[0, :, 0])}"
            assert rel_fro(gv, rv[0, :, 0]) <= 2e-2, f"dV head {h} keys {k0}..: {rel_fro(gv, rv[0, :, 0])}"
            assert np.abs(gv).max() > 0


def _rows_bits(seed, heads):
    """[LQL, heads, DH] bf16 bits, built like _kv_bits over the query axis."""
    base = bf16_bits(bf16_round(
        np.random.default_rng(seed).standard_normal((LQL, DH), dtype=np.float32)))
    out = np.empty((LQL, heads, DH), dtype=np.uint16)
    for h in range(heads):
        s = 991 * h
        out[s:, h, :] = base[:LQL - s]
        out[:s, h, :] = base[LQL - s:]
    return out


LQL = (1 << 21) + 4099  # query rows: LQL * 8 * 128 > 2^31 elements of Q, dO, O, dQ
LKS = 300               # keys, at the last 300 positions of the query range
HQ, HKV = 8, 2          # grouped query heads, 4 per key/value head


def test_pair_past_2_31_query_elements():
    """The query side past 2^31 elements: the keys sit at the last LKS
    positions, so rows before them see nothing (O = 0, LSE = -inf) and the
    last LKS rows, all past the mark, see a causal prefix of them; dK and dV
    then depend on those rows only and are checked exactly.  The LSE merge
    of two partials over halves of the keys runs over the same rows."""
    print(f"case large query pair LQ={LQL} LK={LKS} HQ={HQ} HKV={HKV} d={DH}", flush=True)
    qb, dob = _rows_bits(21, HQ), _rows_bits(22, HQ)
    rng = np.random.default_rng(23)
    k = rand(rng, (1, LKS, HKV, DH), "bf16")
    v = rand(rng, (1, LKS, HKV, DH), "bf16")
    scale = DH ** -0.5
    k0 = LQL - LKS  # kv_start, with q_start = 0
    tail = slice(LQL - LKS, LQL)

    def rows(bits, sl, h0, h1):
        x = (bits[sl, h0:h1, :].astype(np.uint32) << np.uint32(16)).view(np.float32)
        return x.astype(np.float64)[None]

    q_d = torch.from_numpy(qb).to(DEV).view(torch.bfloat16)[None]
    do_d = torch.from_numpy(dob).to(DEV).view(torch.bfloat16)[None]
    k_d, v_d = (torch.from_numpy(x).to(DEV).to(torch.bfloat16) for x in (k, v))
    desc = D.make_desc(1, HQ, HKV, DH, LQL, LKS, 0, k0, True, scale, "bf16")
    o_part = torch.empty(1, LQL, HQ, DH, device=DEV)
    lse = torch.empty(1, HQ, LQL, device=DEV)
    D.dfa_attn_fwd_partial(desc, q_d, k_d, v_d, o_part, lse)
    torch.cuda.synchronize()
    # rows before the keys see nothing
    assert torch.all(o_part[:, :k0] == 0) and torch.all(lse[:, :, :k0] == -float("inf"))
    # the last rows, every head, against the oracle
    qt, dot = rows(qb, tail, 0, HQ), rows(dob, tail, 0, HQ)
    ro, rl = oracle.attention_fwd(qt, k, v, scale, True, LQL - LKS, k0)
    check_o(o_part[:, tail].cpu().numpy().astype(np.float64), ro, "bf16", "O tail")
    check_lse(lse[:, :, tail].cpu().numpy().astype(np.float64), rl, "bf16", "LSE tail")

    # the LSE merge over the same rows: two partials over disjoint halves of
    # the keys merge to the whole (rows that see neither half stay O = 0,
    # LSE = -inf)
    parts = []
    for a0, a1 in ((0, LKS // 2), (LKS // 2, LKS)):
        dsc = D.make_desc(1, HQ, HKV, DH, LQL, a1 - a0, 0, k0 + a0, True, scale, "bf16")
        op = torch.empty(1, LQL, HQ, DH, device=DEV)
        lp = torch.empty(1, HQ, LQL, device=DEV)
        D.dfa_attn_fwd_partial(dsc, q_d, k_d[:, a0:a1].contiguous(), v_d[:, a0:a1].contiguous(),
                               op, lp)
        parts.append((op, lp))
    o_m = torch.empty(1, LQL, HQ, DH, device=DEV, dtype=torch.bfloat16)
    l_m = torch.empty(1, HQ, LQL, device=DEV)
    D.dfa_lse_merge([x[0] for x in parts], [x[1] for x in parts], 1, HQ, LQL, DH, "bf16", o_m, l_m)
    torch.cuda.synchronize()
    del parts
    assert torch.all(o_m[:, :k0] == 0) and torch.all(l_m[:, :, :k0] == -float("inf"))
    check_o(o_m[:, tail].float().cpu().numpy().astype(np.float64), ro, "bf16", "merged O tail",
            stored_bf16=True)
    check_lse(l_m[:, :, tail].cpu().numpy().astype(np.float64), rl, "bf16", "merged LSE tail")
    del o_m, l_m

    # backward from the saved output: the oracle's O (in bf16) and LSE on the
    # rows that see keys, O = 0 and LSE = -inf before them
    o_in = torch.zeros(1, LQL, HQ, DH, device=DEV, dtype=torch.bfloat16)
    o_in[:, tail] = torch.from_numpy(bf16_round(ro.astype(np.float32))).to(DEV).to(torch.bfloat16)
    lse_in = torch.full((1, HQ, LQL), -float("inf"), device=DEV)
    lse_in[:, :, tail] = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    delta = torch.empty(1, HQ, LQL, device=DEV)
    dq = torch.zeros(1, LQL, HQ, DH, device=DEV)
    dk = torch.zeros(1, LKS, HKV, DH, device=DEV)
    dv = torch.zeros(1, LKS, HKV, DH, device=DEV)
    D.dfa_attn_bwd(desc, q_d, k_d, v_d, o_in, lse_in, do_d, delta, True, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(dq[:, :k0] == 0)
    o_t = o_in[:, tail].float().cpu().numpy().astype(np.float64)
    rq, rk, rv = oracle.attention_bwd(qt, k, v, o_t, rl, dot, scale, True, LQL - LKS, k0)
    check_grad(dq[:, tail].cpu().numpy().astype(np.float64), rq, "bf16", "dQ tail")
    check_grad(dk.cpu().numpy().astype(np.float64), rk, "bf16", "dK")
    check_grad(dv.cpu().numpy().astype(np.float64), rv, "bf16", "dV")
