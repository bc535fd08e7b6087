"""The two-stream exchange emulation ([DistFlashAttn §3.2]: key/value
prefetch on a separate stream, overlapped with compute) gives the oracle's
partials, and bitwise the results of the plain forward, for owners and for
helpers whose results are sent back to their owners."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd.runner import ChunkedCausalAttention

from _util import check_lse, check_o, rand, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(dfa_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("p,c,window", [(5, 160, 0), (4, 128, 0), (4, 128, 200)])
def test_overlapped_worker_forward_is_bitwise_plain(p, c, window):
    print(f"case overlap {p} {c} {window}", flush=True)
    rng = np.random.default_rng(p * 10 + c)
    att = ChunkedCausalAttention(p, c, 1, 4, 2, 128, "bf16", window=window)
    qh = [rand(rng, att.q_shape(), "bf16") for _ in range(p)]
    kh = [rand(rng, att.kv_shape(), "bf16") for _ in range(p)]
    vh = [rand(rng, att.kv_shape(), "bf16") for _ in range(p)]
    q, k, v = ({a: to_dev(x[a], "bf16") for a in range(p)} for x in (qh, kh, vh))
    ref = {(it[2], it[3]): att.new_partial() for it in att.items}
    att.forward_items(att.items, q, k, v, ref)
    for overlap in (True, False):
        got = {key: (torch.full_like(o, 7.0), torch.full_like(l_, 7.0)) for key, (o, l_) in ref.items()}
        for w in range(p):
            att.forward_worker_overlapped(w, q, k, v, got, overlap=overlap)
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(got[key][0], ref[key][0]), (overlap, key)
            assert torch.equal(got[key][1], ref[key][1]), (overlap, key)
            a, cc = key
            ro, rl = oracle.attention_fwd(qh[a], kh[cc], vh[cc], att.scale, True, a * c, cc * c,
                                          window=window)
            check_o(to_np(got[key][0]), ro, "bf16", f"overlapped O_part{key}")
            check_lse(to_np(got[key][1]), rl, "bf16", f"overlapped LSE_part{key}")
