"""The autograd binding and the checkpoint placements of the Llama-shaped
layer ([DistFlashAttn §3.3]: checkpointing the attention output avoids the
attention forward's recomputation "without numerical differences").

* `chunked_attention` through torch autograd equals the float64 oracle's
  whole-sequence forward and backward (bf16 tolerances).
* One layer's output and every gradient are bitwise identical under the
  three placements, and the attention forward runs once per step with
  "none" and "remat" but twice with layer-boundary checkpointing.
"""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import autograd as A
from long_context_exact_amd.layer import MODES, LlamaLayer
from long_context_exact_amd.runner import ChunkedCausalAttention

from _util import DEV, check_grad, check_o, rand, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("p,c,hq,hkv,d,window", [(3, 128, 4, 2, 64, 0), (4, 96, 8, 1, 128, 0),
                                                   (3, 128, 4, 4, 128, 100)])
def test_autograd_function_matches_oracle(p, c, hq, hkv, d, window):
    print(f"case autograd {p} {c} {hq} {hkv} {d} {window}", flush=True)
    rng = np.random.default_rng(p * 100 + c)
    n = p * c
    q, k, v = (rand(rng, (1, n, h, d), "bf16") for h in (hq, hkv, hkv))
    do = rand(rng, (1, n, hq, d), "bf16")
    att = ChunkedCausalAttention(p, c, 1, hq, hkv, d, "bf16", window=window)
    tq, tk, tv = (torch.from_numpy(x).to(DEV).to(torch.bfloat16).requires_grad_(True)
                  for x in (q, k, v))
    o = A.chunked_attention(tq, tk, tv, att)
    o.backward(torch.from_numpy(do).to(DEV).to(torch.bfloat16))
    ro, rl = oracle.attention_fwd(q, k, v, att.scale, True, 0, 0, window=window)
    check_o(to_np(o), ro, "bf16", stored_bf16=True)
    rq, rk, rv = oracle.attention_bwd(q, k, v, to_np(o), rl, do, att.scale, True, 0, 0,
                                      window=window)
    for g, r, name in ((tq.grad, rq, "dQ"), (tk.grad, rk, "dK"), (tv.grad, rv, "dV")):
        check_grad(to_np(g), r, "bf16", name)


def test_checkpoint_placements_change_no_numbers():
    print("case layer modes", flush=True)
    att = ChunkedCausalAttention(3, 128, 1, 4, 2, 64, "bf16")
    layer = LlamaLayer(att, 256, 512, DEV, seed=3)
    gen = torch.Generator(device="cpu").manual_seed(9)
    x0 = torch.randn(1, 384, 256, generator=gen).to(DEV, torch.bfloat16)
    dy = torch.randn(1, 384, 256, generator=gen).to(DEV, torch.bfloat16)
    out = {}
    for mode in MODES:
        layer.zero_grad(set_to_none=True)
        x = x0.clone().requires_grad_(True)
        calls = A.FORWARD_CALLS[0]
        y = layer(x, mode)
        y.backward(dy)
        torch.cuda.synchronize()
        out[mode] = {"y": y.detach().clone(), "x": x.grad.clone(),
                     "p": [q.grad.clone() for q in layer.parameters()],
                     "fwd": A.FORWARD_CALLS[0] - calls}
    assert out["none"]["fwd"] == 1 and out["remat"]["fwd"] == 1 and out["layer"]["fwd"] == 2
    for mode in ("layer", "remat"):
        assert torch.equal(out[mode]["y"], out["none"]["y"]), mode
        assert torch.equal(out[mode]["x"], out["none"]["x"]), mode
        for a, b in zip(out[mode]["p"], out["none"]["p"]):
            assert torch.equal(a, b), mode
    assert all(torch.isfinite(g).all() for g in out["remat"]["p"])
    assert float(out["remat"]["x"].float().abs().max()) > 0
