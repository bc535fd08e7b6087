"""Time one worker's forward items with the per-step exchange emulated on a
second stream ([DistFlashAttn §3.2]: key/value prefetch overlapped with the
attention computation), against the same copies in line on one stream and
against no copies at all:

    python -m long_context_exact_amd.overlap_bench [--workload gqa64x8_512k_w15]

On one GPU the "transfer" is a device-to-device copy at HBM speed, not an
xGMI link, so this shows the mechanism and its cost, not the pages' 1.32x.
"""

from __future__ import annotations

import argparse
import json

import torch

from .runner import ChunkedCausalAttention
from .synth import WORKLOADS


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="gqa64x8_512k_w15")
    ap.add_argument("--workers", default="15,0", help="which workers' shares to time")
    ap.add_argument("--steps", type=int, default=3)
    args = ap.parse_args()
    w = WORKLOADS[args.workload]
    att = ChunkedCausalAttention(w.workers, w.chunk, w.batch, w.heads_q, w.heads_kv, w.head_dim,
                                 w.dtype, window=w.window)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cpu").manual_seed(7)
    res = {"metric": "one worker's forward items: ms with the exchange overlapped / in line / absent",
           "workload": w.name, "workers": {}}
    for wk in (int(x) for x in args.workers.split(",")):
        its = att.items_of_worker(wk)
        need_q = sorted({it[2] for it in its} | {wk})
        need_kv = sorted({it[3] for it in its} | {wk})
        mk = lambda shape: torch.randn(*shape, generator=gen).to("cuda", td)  # noqa: E731
        q = {a: mk(att.q_shape()) for a in need_q}
        k = {c: mk(att.kv_shape()) for c in need_kv}
        v = {c: mk(att.kv_shape()) for c in need_kv}
        partials = {(it[2], it[3]): att.new_partial() for it in its}
        out = {}
        for mode in ("overlapped", "in_line", "no_copies"):
            def run():
                if mode == "no_copies":
                    att.forward_items(its, q, k, v, partials)
                else:
                    att.forward_worker_overlapped(wk, q, k, v, partials, overlap=mode == "overlapped")
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                run()
            e1.record()
            torch.cuda.synchronize()
            out[mode] = round(e0.elapsed_time(e1) / args.steps, 3)
        moved = sum((q[it[2]].numel() * q[it[2]].element_size() if it[2] != wk else
                     (2 * k[it[3]].numel() * k[it[3]].element_size() if it[3] != wk else 0))
                    for it in its)
        res["workers"][wk] = {"items": len(its), "bytes_received": moved, "ms": out,
                              "exposed_copy_ms": round(out["overlapped"] - out["no_copies"], 3)}
        del q, k, v, partials
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
