"""Time one Llama-7B-shaped layer's forward + backward under the three
checkpoint placements of `layer.py` ([DistFlashAttn §3.3]):

    python -m long_context_exact_amd.layer_bench [--workers 8 --chunk 8192 --steps 3]

Prints one JSON line: ms per training step of the layer for "none",
"layer" (layer-boundary checkpointing) and "remat" (checkpoint at the
attention output), the attention forward passes each ran per step, the
attention forward time on its own, and each mode's peak device memory.
Synthetic input x ~ N(0, 1), random weights.
"""

from __future__ import annotations

import argparse
import json

import torch

from . import autograd as A
from .layer import MODES, layer_flops, llama7b_layer


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=8)
    ap.add_argument("--chunk", type=int, default=8192)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    args = ap.parse_args()
    layer = llama7b_layer(args.workers, args.chunk)
    n = args.workers * args.chunk
    gen = torch.Generator(device="cpu").manual_seed(1)
    x0 = torch.randn(1, n, 4096, generator=gen).to("cuda", torch.bfloat16)
    dy = torch.randn(1, n, 4096, generator=gen).to("cuda", torch.bfloat16) * 1e-2
    res = {"metric": "Llama-7B layer fwd+bwd ms per step by checkpoint placement",
           "config": {"tokens": n, "workers": args.workers, "chunk": args.chunk, "hidden": 4096,
                      "heads": 32, "head_dim": 128, "intermediate": 11008, "dtype": "bf16"},
           "modes": {}}
    for mode in MODES:
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        times = []
        for i in range(args.warmup + args.steps):
            x = x0.clone().requires_grad_(True)
            layer.zero_grad(set_to_none=True)
            calls0 = A.FORWARD_CALLS[0]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            y = layer(x, mode)
            y.backward(dy)
            e1.record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                times.append(e0.elapsed_time(e1))
            fwd_calls = A.FORWARD_CALLS[0] - calls0
            del y, x
        res["modes"][mode] = {"ms_per_step": round(sum(times) / len(times), 3),
                              "attention_forwards_per_step": fwd_calls,
                              "peak_mem_gib": round(torch.cuda.max_memory_allocated() / 2**30, 2)}
    with torch.no_grad():
        q, k, v = layer.pre_attn(x0)
        A.attention_forward(layer.att, q, k, v)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            A.attention_forward(layer.att, q, k, v)
        e1.record()
        torch.cuda.synchronize()
    gemm, attn = layer_flops(layer.att, 4096, 11008)
    res["attention_forward_ms"] = round(e0.elapsed_time(e1) / args.steps, 3)
    res["forward_flop"] = {"gemm": gemm, "attention": attn}
    m = res["modes"]
    res["remat_speedup_over_layer"] = round(m["layer"]["ms_per_step"] / m["remat"]["ms_per_step"], 4)
    res["saved_ms_per_layer"] = round(m["layer"]["ms_per_step"] - m["remat"]["ms_per_step"], 3)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
