"""Run each compute kernel of one fully visible chunk pair back to back for a
few seconds, one kernel at a time, so that an outside monitor (for instance
`amd-smi metric -p -c` sampled meanwhile) sees the board power and shader
clock each kernel settles at.  The pair is the headline shape: a 32768-token
query chunk against an earlier 32768-token key/value chunk, 64 query and 8
key/value heads of 128, bf16.

    python -m long_context_exact_amd.kernel_loop [--seconds 4] [--kernels fwd,dkdv,dq]

Prints one JSON line per kernel with the wall-clock interval it ran in, the
number of launches and the mean time per launch.  The backward kernels run
alone through the library's test-support entry point `dfa_test_bwd_part`.
"""

from __future__ import annotations

import argparse
import json
import time

import torch

from . import dfa as D


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--seconds", type=float, default=4.0)
    ap.add_argument("--kernels", default="fwd,dkdv,dq")
    ap.add_argument("--pause", type=float, default=1.0, help="idle seconds between kernels")
    args = ap.parse_args(argv)

    c, hq, hkv, dh, dev = 32768, 64, 8, 128, "cuda"
    g = torch.Generator(device=dev).manual_seed(5)
    q, do = (torch.randn(1, c, hq, dh, device=dev, generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(1, c, hkv, dh, device=dev, generator=g).to(torch.bfloat16) for _ in range(2))
    desc = D.make_desc(1, hq, hkv, dh, c, c, c, 0, True, dh ** -0.5, "bf16")  # fully visible
    o = torch.empty(1, c, hq, dh, device=dev)
    lse = torch.empty(1, hq, c, device=dev)
    D.dfa_attn_fwd_partial(desc, q, k, v, o, lse)
    delta = torch.empty_like(lse)
    dq = torch.zeros(1, c, hq, dh, device=dev)
    dk = torch.zeros(1, c, hkv, dh, device=dev)
    dv = torch.zeros_like(dk)
    D.dfa_attn_bwd(desc, q, k, v, o.to(torch.bfloat16), lse, do, delta, True, dq, dk, dv)
    torch.cuda.synchronize()
    runs = {"fwd": lambda: D.dfa_attn_fwd_partial(desc, q, k, v, o, lse),
            "dkdv": lambda: D.dfa_test_bwd_part(desc, q, k, v, lse, do, delta, dq, dk, dv, 1),
            "dq": lambda: D.dfa_test_bwd_part(desc, q, k, v, lse, do, delta, dq, dk, dv, 2)}
    for name in args.kernels.split(","):
        fn = runs[name]
        fn()
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        while time.time() - t0 < args.seconds:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
            n += 8
        t1 = time.time()
        print(json.dumps({"kernel": name, "t0": t0, "t1": t1, "launches": n,
                          "ms_per_launch": (t1 - t0) * 1e3 / n}), flush=True)
        time.sleep(args.pause)


if __name__ == "__main__":
    main()
