"""Time one worker's forward items with the per-step exchange emulated on a
second stream ([DistFlashAttn §3.2]: key/value prefetch overlapped with the
attention computation), against the same transfers in line on one stream,
against no transfers at all, and the transfers alone:

    python -m long_context_exact_amd.overlap_bench [--workload gqa64x8_512k_w15]

Each transfer is a DMA-engine copy (dfa_chunk_transfer), so like a link
transfer it takes no compute units.  The modes are timed in turn over
several rounds (one pass of each per round) and the medians reported, so
that a drift of the power-limited clock does not favour one mode.  On one
GPU the copy engines move a chunk far faster than the pages' links did, so
this shows the mechanism and what it hides, not the pages' 1.32x.
"""

from __future__ import annotations

import argparse
import json
import statistics

import torch

from . import dfa
from .runner import ChunkedCausalAttention
from .synth import WORKLOADS


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="gqa64x8_512k_w15")
    ap.add_argument("--workers", default="15,0", help="which workers' shares to time")
    ap.add_argument("--rounds", type=int, default=5)
    args = ap.parse_args()
    w = WORKLOADS[args.workload]
    att = ChunkedCausalAttention(w.workers, w.chunk, w.batch, w.heads_q, w.heads_kv, w.head_dim,
                                 w.dtype, window=w.window)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cpu").manual_seed(7)
    res = {"metric": "one worker's forward items: median ms with the exchange overlapped / in "
                     "line / absent, and the transfers alone",
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

        def copies_only():
            """The same transfers, issued as the worker would, without compute:
            a helper receives the owner's queries and sends its (O, LSE) back."""
            comm = torch.cuda.current_stream()
            for it in its:
                a, c = it[2], it[3]
                if a != wk:
                    dfa.dfa_chunk_transfer(slot_q, q[a], comm)
                    for dst, src in zip(ret, partials[(a, c)]):
                        dfa.dfa_chunk_transfer(dst, src, comm)
                elif c != wk:
                    dfa.dfa_chunk_transfer(slot_k, k[c], comm)
                    dfa.dfa_chunk_transfer(slot_v, v[c], comm)

        slot_q, slot_k, slot_v = (torch.empty_like(q[wk]), torch.empty_like(k[wk]),
                                  torch.empty_like(v[wk]))
        ret = att.new_partial()
        runs = {
            "overlapped": lambda: att.forward_worker_overlapped(wk, q, k, v, partials, True),
            "in_line": lambda: att.forward_worker_overlapped(wk, q, k, v, partials, False),
            "no_copies": lambda: att.forward_items(its, q, k, v, partials),
            "copies_only": copies_only,
        }
        for fn in runs.values():  # warm-up
            fn()
        torch.cuda.synchronize()
        times = {m: [] for m in runs}
        for _ in range(args.rounds):
            for mode, fn in runs.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times[mode].append(e0.elapsed_time(e1))
        out = {m: round(statistics.median(t), 3) for m, t in times.items()}
        moved = sum((q[it[2]].numel() * q[it[2]].element_size() if it[2] != wk else
                     (2 * k[it[3]].numel() * k[it[3]].element_size() if it[3] != wk else 0))
                    for it in its)
        res["workers"][wk] = {"items": len(its), "bytes_received": moved, "median_ms": out,
                              "rounds": args.rounds,
                              "exposed_copy_ms": round(out["overlapped"] - out["no_copies"], 3),
                              "in_line_copy_ms": round(out["in_line"] - out["no_copies"], 3)}
        del q, k, v, partials, slot_q, slot_k, slot_v, ret
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
