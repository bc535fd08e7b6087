"""The library keeps no state between calls: its scratch (the forward's
transposed V, dK/dV's row-split partials) is the caller's workspace.  Calls
with their own workspaces may overlap on different streams, or be issued
from different host threads onto one stream; every result must equal, bit
for bit, the same call run alone."""

import threading

import numpy as np
import pytest
import torch

from long_context_exact_amd import dfa as D

from _util import DEV, rand, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(seed, lq, lk):
    """A pair whose dK/dV splits rows (a short key range against many rows)."""
    rng = np.random.default_rng(seed)
    hq, hkv, dh = 8, 2, 128
    t = {n: to_dev(rand(rng, s, "bf16"), "bf16") for n, s in
         (("q", (1, lq, hq, dh)), ("k", (1, lk, hkv, dh)), ("v", (1, lk, hkv, dh)),
          ("do", (1, lq, hq, dh)))}
    desc = D.make_desc(1, hq, hkv, dh, lq, lk, lk, 0, True, dh ** -0.5, "bf16")
    return desc, t


def _run(desc, t, stream, ws=None):
    """Forward then backward of one pair on `stream`; ws: (forward,
    backward) workspaces, or None for the binding to take them per call."""
    with torch.cuda.stream(stream):
        lq, hq, dh = desc.len_q, desc.heads_q, desc.head_dim
        o = torch.empty(1, lq, hq, dh, device=DEV)
        lse = torch.empty(1, hq, lq, device=DEV)
        D.dfa_attn_fwd_partial(desc, t["q"], t["k"], t["v"], o, lse, stream=stream,
                               workspace=None if ws is None else ws[0])
        ob = o.to(torch.bfloat16)
        delta = torch.empty_like(lse)
        dq = torch.zeros_like(o)
        dk = torch.zeros(1, desc.len_kv, desc.heads_kv, dh, device=DEV)
        dv = torch.zeros_like(dk)
        D.dfa_attn_bwd(desc, t["q"], t["k"], t["v"], ob, lse, t["do"], delta, True, dq, dk, dv,
                       stream=stream, workspace=None if ws is None else ws[1])
    return o, lse, dq, dk, dv


def _workspaces(desc, stream):
    with torch.cuda.stream(stream):
        return tuple(torch.empty(max(1, D.dfa_attn_workspace_size(desc, op)), dtype=torch.uint8,
                                 device=DEV) for op in (D.DFA_OP_FWD, D.DFA_OP_BWD))


def test_two_streams_match_each_call_alone():
    print("case two streams", flush=True)
    cases = [_case(1, 8192, 512), _case(2, 6144, 768)]
    alone = []
    for desc, t in cases:
        s = torch.cuda.Stream()
        alone.append(_run(desc, t, s))
        torch.cuda.synchronize()
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):  # interleaved: both streams' calls in flight together
        r0 = _run(*cases[0], s0)
        r1 = _run(*cases[1], s1)
        torch.cuda.synchronize()
        for got, want in ((r0, alone[0]), (r1, alone[1])):
            for x, y in zip(got, want):
                assert torch.equal(x, y)


def test_two_threads_one_stream_match_each_call_alone():
    """Two host threads issue pairs of the same shape onto one stream, each
    with its own workspaces; their enqueues interleave, results must not."""
    print("case two threads one stream", flush=True)
    cases = [_case(3, 8192, 512), _case(4, 8192, 512)]
    assert D.dfa_attn_workspace_size(cases[0][0], D.DFA_OP_BWD) > 0  # the row split runs
    s = torch.cuda.Stream()
    alone = []
    for desc, t in cases:
        alone.append(_run(desc, t, s, _workspaces(desc, s)))
        torch.cuda.synchronize()
    ws = [_workspaces(desc, s) for desc, _ in cases]
    got = [None, None]
    start = threading.Barrier(2)

    def worker(i):
        torch.cuda.set_device(0)
        start.wait()
        got[i] = [_run(*cases[i], s, ws[i]) for _ in range(4)]

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    for i in range(2):
        assert got[i] is not None
        for rep in got[i]:
            for x, y in zip(rep, alone[i]):
                assert torch.equal(x, y)
