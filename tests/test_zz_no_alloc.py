"""dfa_attn_fwd_partial_noalloc (scratch in the library's fixed per-device
array, nothing allocated) against dfa_attn_fwd_partial (scratch in a caller
workspace) through the C ABI: bitwise-equal outputs on two calls in a row,
the second with a smaller input, plus the capacity limit."""

import numpy as np
import pytest
import torch

from long_context_exact_amd import dfa as D

from _util import DEV, case_seed, rand, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(seed, b, hq, hkv, dh, lq, lk, q0, k0, window=0):
    rng = np.random.default_rng(seed)
    desc = D.make_desc(b, hq, hkv, dh, lq, lk, q0, k0, True, dh ** -0.5, "bf16", window)
    t = [to_dev(rand(rng, (b, lq, hq, dh), "bf16"), "bf16")] + \
        [to_dev(rand(rng, (b, lk, hkv, dh), "bf16"), "bf16") for _ in range(2)]
    return desc, t


def _outputs(desc):
    o = torch.full((desc.batch, desc.len_q, desc.heads_q, desc.head_dim), float("nan"),
                   device=DEV)
    lse = torch.full((desc.batch, desc.heads_q, desc.len_q), float("nan"), device=DEV)
    return o, lse


def test_noalloc_forward_matches_workspace_forward_twice():
    print("case no-alloc forward: large then smaller pair", flush=True)
    cases = [_pair(case_seed("noalloc-1"), 1, 64, 8, 128, 4096, 32768, 15 * 32768 + 28672,
                   14 * 32768),                                           # 64 MiB of V^T: the limit
             _pair(case_seed("noalloc-2"), 2, 6, 3, 64, 300, 333, 500, 400, 150)]
    assert D.dfa_attn_workspace_size(cases[0][0], D.DFA_OP_FWD) == 64 << 20
    for desc, (q, k, v) in cases:
        want = _outputs(desc)
        D.dfa_attn_fwd_partial(desc, q, k, v, *want)
        got = _outputs(desc)
        D.dfa_attn_fwd_partial_noalloc(desc, q, k, v, *got)
        torch.cuda.synchronize()
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])


def test_noalloc_forward_rejects_scratch_past_its_limit():
    desc = D.make_desc(1, 8, 8, 128, 64, 32768)          # 8 heads x 32768 keys: 64 MiB
    assert D.dfa_attn_workspace_size(desc, D.DFA_OP_FWD) == 64 << 20
    big = D.make_desc(1, 8, 8, 128, 64, 32769)           # one key more: past the limit
    q = torch.zeros(1, 64, 8, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, 32769, 8, 128, dtype=torch.bfloat16, device=DEV)
    o, lse = _outputs(big)
    with pytest.raises(D.DfaError, match="fixed scratch holds") as e:
        D.dfa_attn_fwd_partial_noalloc(big, q, kv, kv, o, lse)
    assert e.value.status == D.DFA_ERR_CAPACITY
