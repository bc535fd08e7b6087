"""GPU parity of the backward of diagonal chunk pairs run as row bands.

A diagonal pair (query and key chunk the same tokens) of whole 256-key
blocks whose rows the kernel does not split has its dK/dV computed in two
launches: each key block's own rows in the masked kernel (with a window that
is a multiple of 32 rows, at least 512 and shorter than the chunk, paired in
the same launch with the rows at the window's edge, each wave taking the one
of the two tiles it sees), and the rows in between (which see every key of
the block) in the mask-free one.
Every gradient is compared element by element with the float64 oracle, on
shapes that take the banded path and on one that just misses it (a window
that is not a multiple of 32 rows), and repeated runs must agree bit for
bit."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import dfa as D

from _util import DEV, check_grad, rand, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("b,l,start,hq,hkv,dh,win,launches", [
    (2, 2048, 0, 16, 16, 128, 0, 2),       # own rows masked, the rest mask-free
    (2, 2048, 0, 16, 16, 128, 512, 2),     # paired bands, the smallest window that bands
    (2, 2048, 4096, 16, 16, 64, 800, 2),   # head_dim 64, non-zero chunk start, 25-tile window
    (16, 2048, 0, 8, 2, 64, 0, 2),         # four query heads per key/value head
    (2, 2560, 0, 16, 16, 128, 1024, 2),    # late blocks' window-edge tiles cut by the chunk's end
    (8, 1024, 0, 32, 8, 128, 544, 2),      # window-edge tiles of a 17-tile window, GQA 4
    (2, 2048, 0, 16, 16, 128, 2048, 2),    # window as long as the chunk: own rows alone
    (2, 2048, 0, 16, 16, 128, 500, 1),     # not a multiple of 32 rows: one masked launch
])
def test_banded_diagonal_pair_backward(b, l, start, hq, hkv, dh, win, launches):
    print(f"case banded {b} {l} {start} {hq} {hkv} {dh} {win}", flush=True)
    rng = np.random.default_rng(b * 7 + l * 131 + hq * 17 + dh + win)
    scale = dh ** -0.5
    q = rand(rng, (b, l, hq, dh), "bf16")
    k = rand(rng, (b, l, hkv, dh), "bf16")
    v = rand(rng, (b, l, hkv, dh), "bf16")
    d_o = rand(rng, (b, l, hq, dh), "bf16")
    desc = D.make_desc(b, hq, hkv, dh, l, l, start, start, True, scale, "bf16", window=win)
    assert D.dfa_test_bwd_launches(desc, 1) == launches  # the path this case is for
    ro, rl = oracle.attention_fwd(q, k, v, scale, True, start, start, window=win)
    o_in = to_dev(ro.astype(np.float32), "bf16")
    lse_in = torch.from_numpy(rl.astype(np.float32)).to(DEV)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o_in), rl, d_o, scale, True, start, start,
                                      window=win)
    qd, kd, vd, dod = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(d_o, "bf16")
    runs = []
    for _ in range(2):
        delta = torch.empty_like(lse_in)
        dq = torch.zeros(b, l, hq, dh, device=DEV)
        dk = torch.zeros(b, l, hkv, dh, device=DEV)
        dv = torch.zeros(b, l, hkv, dh, device=DEV)
        D.dfa_attn_bwd(desc, qd, kd, vd, o_in, lse_in, dod, delta, True, dq, dk, dv)
        torch.cuda.synchronize()
        runs.append([to_np(x) for x in (dq, dk, dv)])
    for g, r, n in zip(runs[0], (rq, rk, rv), ("dQ", "dK", "dV")):
        check_grad(g, r, "bf16", n)
    for x, y in zip(runs[0], runs[1]):
        assert np.array_equal(x, y)
