#!/usr/bin/env python3
"""Throughput of the chunked causal attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
inputs already resident in HBM.  For a worker-share workload (default: the
grouped-query 64/8-head, head_dim 128 case at a 32768-token chunk, worker
15 of 16 on a 524288-token sequence) the step is that worker's share of the
load-balanced schedule:
    its 9 forward pairs (1 diagonal + 8 full),
    the LSE merge of all 16 partials of its query chunk (the 7 computed by
    helpers are inputs, prepared before timing, as received messages),
    the backward of its 9 pairs from the merged O and LSE (delta once),
including zeroing the fp32 gradient accumulators.  Whole-sequence workloads
run every pair, every merge and (if any) every backward.

Prints ONE JSON line.  TFLOP/s counts only unmasked (query, key) pairs:
forward 4*d and backward 10*d FLOP per pair per query head.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s (1 GPU) at 32K chunk; % of bf16 MFMA peak"
# Peaks of the arithmetic each input dtype runs in on MI355X: bf16 inputs on
# dense bf16 MFMA; fp32 inputs on the exact path, fp64 on the vector ALU.
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 78.6}
ARITH_DTYPE = {"bf16": "bf16", "f32": "f64"}


# Profiler names of the kernels the default build launches for bf16 head_dim 128.
KERNEL_NAMES = {"fwd": "fwd_bf16_kernel", "dkdv": "dkdv_bf16_kernel", "dq": "dq_bf16_kernel"}
# fp32 inputs run the exact kernels (one wave per row, fp64 on the vector ALU, no MFMA)
KERNEL_NAMES_F32 = {"fwd": "fwd_f32_kernel", "dkdv": "dkdv_f32_kernel", "dq": "dq_f32_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {"fwd_bf16_kernel": ("fwd_mfma.hip", "transpose.hip"),
                  "dkdv_bf16_kernel": ("dkdv_mfma.hip", "bwd_common.hpp"),
                  "dq_bf16_kernel": ("dq_mfma.hip", "bwd_common.hpp")}


def source_digest(name: str) -> str:
    import hashlib
    csrc = os.path.join(ROOT, "long_context_exact_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name] + ("common.hpp",):
        h.update(open(os.path.join(csrc, f), "rb").read())
    # the compiler options are part of the kernel too
    h.update(open(os.path.join(ROOT, "long_context_exact_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


def traffic_of(name: str, launches: int, workload: str):
    """HBM bytes per launch of `name` from the committed counter summary (the
    total, the FETCH and WRITE parts and what they were averaged over), or
    None if there is none, it was taken on another workload, or the kernel's
    sources changed since it was taken."""
    try:
        doc = json.load(open(TRAFFIC_FILE))
        t = doc["kernels"][name]
    except (OSError, KeyError, ValueError):
        return None
    if doc.get("workload") != workload or t.get("source_digest") != source_digest(name):
        return None
    return {"bytes_per_launch": t["bytes_per_launch"], "fetch": t["fetch_bytes_per_launch"],
            "write": t["write_bytes_per_launch"], "workload": t["workload"]}


def pairs_of(kind: int, c: int) -> int:
    return c * (c + 1) // 2 if kind == 0 else c * c


def item_keys(item, c: int, n_global: int):
    """(first key position, end position, window) of an item: the global
    prefix (kv chunk -1, no window), chunk 0 past the global prefix, or the
    whole kv chunk."""
    kc = item[3]
    if kc == -1:
        return 0, n_global, 0
    return (n_global if kc == 0 else kc * c), (kc + 1) * c, None


def visible_pairs(item, c: int, window: int, n_global: int = 0) -> int:
    """(query, key) pairs of an item that the mask keeps: the causal prefix
    of its keys, cut to the keys less than `window` positions behind the
    query (the global item's keys are never cut)."""
    k0, k1, win = item_keys(item, c, n_global)
    win = window if win is None else win
    if win <= 0 and k0 == item[3] * c and k1 - k0 == c:
        return pairs_of(item[4], c)
    import numpy as np
    qpos = item[2] * c + np.arange(c, dtype=np.int64)
    hi = np.minimum(k1 - 1, qpos)                                  # last visible key
    lo = k0 if win <= 0 else np.maximum(k0, qpos - win + 1)        # first visible key
    return int(np.maximum(hi - lo + 1, 0).sum())


def gen_inputs(w, chunks_q, chunks_kv, backward):
    """Seeded per-chunk inputs (numpy float32, bf16-exact), drawn in threads."""
    import concurrent.futures as cf

    from long_context_exact_amd.synth import TENSOR_DO, TENSOR_K, TENSOR_Q, TENSOR_V

    jobs = [(TENSOR_Q, a) for a in chunks_q] + [(TENSOR_K, c) for c in chunks_kv] + \
           [(TENSOR_V, c) for c in chunks_kv] + ([(TENSOR_DO, a) for a in chunks_q] if backward else [])
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        arrs = list(ex.map(lambda j: w.chunk_input(*j), jobs))
    out = {0: {}, 1: {}, 2: {}, 3: {}}
    for (tid, c), x in zip(jobs, arrs):
        out[tid][c] = x
    return out


def cpu_baseline(w, host, worker, budget_s, kv_lo):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: the last R query rows of the measured query chunk, query head 0,
    over their whole causal prefix, forward + backward.  kv_lo: the lowest
    key chunk of the owner's chunk pairs (the global item aside)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    a = worker if worker >= 0 else w.workers - 1
    c = w.chunk
    # the rows' keys as contiguous position ranges (k0, k1, window): the
    # window's chunks, and with global tokens also the global prefix
    g = w.n_global
    ranges = [((g if kv_lo == 0 else kv_lo * c), (a + 1) * c, w.window)]
    if g > 0:
        ranges.insert(0, (0, g, 0))

    def keys(k0, k1, tid):
        chunks = [host[tid][j][:, :, :1] for j in range(k0 // c, (k1 - 1) // c + 1)]
        return np.concatenate(chunks, axis=1)[:, k0 % c:k0 % c + (k1 - k0)].astype(np.float64)

    parts = [(keys(k0, k1, 1), keys(k0, k1, 2), k0, win) for k0, k1, win in ranges]

    def run(r):
        q = host[0][a][:, c - r:, :1].astype(np.float64)
        do = host[3][a][:, c - r:, :1].astype(np.float64) if 3 in host and a in host[3] else \
            np.ones_like(q)
        q0 = a * c + c - r
        t0 = time.perf_counter()
        outs = [oracle.attention_fwd(q, kp, vp, w.scale, True, q0, k0, window=win)
                for kp, vp, k0, win in parts]
        o, lse = outs[0] if len(outs) == 1 else oracle.lse_merge([x[0] for x in outs],
                                                                  [x[1] for x in outs])
        t1 = time.perf_counter()
        for kp, vp, k0, win in parts:
            oracle.attention_bwd(q, kp, vp, o, lse, do, w.scale, True, q0, k0, window=win)
        t2 = time.perf_counter()
        pos = q0 + np.arange(r)
        pairs = 0
        for kp, _, k0, win in parts:
            hi = np.minimum(k0 + kp.shape[1] - 1, pos)
            lo = k0 if win <= 0 else np.maximum(k0, pos - win + 1)
            pairs += int(np.maximum(hi - lo + 1, 0).sum())
        return t2 - t0, pairs * 14 * w.head_dim, (t1 - t0, pairs * 4 * w.head_dim), \
            (t2 - t1, pairs * 10 * w.head_dim)

    # grow the sample until one run takes most of the budget (cost is not
    # linear in r at small r, so a single extrapolation undershoots)
    r = 8
    dt, flops, fw, bw = run(r)
    for _ in range(5):
        if dt >= 0.6 * budget_s or r >= c:
            break
        r = int(min(c, max(r + 8, r * min(8.0, budget_s / max(dt, 1e-3)))))
        dt, flops, fw, bw = run(r)
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = sum(i.get("num_threads", 0) for i in blas)
    lib = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas) or "unknown"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads or 1),
            "kind": "oracle",
            "sample": f"float64 numpy oracle ({lib}), fwd+bwd of the last {r} query rows of chunk "
                      f"{a}, query head 0, over every key they see (keys "
                      f"{', '.join(f'{k0}..{k1 - 1}' for k0, k1, _ in ranges)}"
                      f"{f', window {w.window}' if w.window else ''}"
                      f"{f', the first {g} global' if g else ''}); "
                      f"{dt:.1f} s, {flops:.3e} algorithmic FLOP",
            "fwd_gflops": round(fw[1] / fw[0] / 1e9, 2), "bwd_gflops": round(bw[1] / bw[0] / 1e9, 2)}


# Bytes of the device-to-device copy every run makes before timing: a plain
# copy kernel of known size, whose FETCH_SIZE / WRITE_SIZE readings in the same
# profiling run scale the attention kernels' readings to bytes.
REFERENCE_COPY_BYTES = 1 << 30


def reference_copy():
    import torch
    src = torch.ones(REFERENCE_COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa64x8_512k_w15")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the schedule's "
              "workers are emulated as work items on one device); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_exact_amd import dfa
    from long_context_exact_amd.runner import ChunkedCausalAttention
    from long_context_exact_amd.synth import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = "cuda"
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    att = ChunkedCausalAttention(w.workers, w.chunk, w.batch, w.heads_q, w.heads_kv, w.head_dim,
                                 w.dtype, True, window=w.window, n_global=w.n_global)
    if w.share_of >= 0:
        owners = [w.share_of]
        timed = att.items_of_worker(w.share_of)
        assert all(it[5] == w.share_of for it in timed)
        merged = {w.share_of: att.items_of_owner(w.share_of)}
    else:
        owners = list(range(w.workers))
        timed = att.items
        merged = {a: att.items_of_owner(a) for a in owners}
    kv_needed = sorted({att.kv_rows(it[3])[0] for its in merged.values() for it in its})

    reference_copy()
    t0 = time.perf_counter()
    host = gen_inputs(w, owners, kv_needed, w.backward)
    q = {a: torch.from_numpy(host[0][a]).to(dev).to(td) for a in owners}
    k = {c: torch.from_numpy(host[1][c]).to(dev).to(td) for c in kv_needed}
    v = {c: torch.from_numpy(host[2][c]).to(dev).to(td) for c in kv_needed}
    d_o = {a: torch.from_numpy(host[3][a]).to(dev).to(td) for a in owners} if w.backward else {}
    gen_s = time.perf_counter() - t0

    partials = {(it[2], it[3]): att.new_partial(dev) for its in merged.values() for it in its}
    helpers = [it for its in merged.values() for it in its if it not in timed]
    att.forward_items(helpers, q, k, v, partials)          # received messages: untimed
    o = {a: torch.empty(att.q_shape(), dtype=td, device=dev) for a in owners}
    lse = {a: torch.empty(att.lse_shape(), device=dev) for a in owners}
    delta = {a: torch.empty(att.lse_shape(), device=dev) for a in owners}
    dq = {a: torch.zeros(att.q_shape(), device=dev) for a in owners}
    own_kv = sorted({att.kv_rows(it[3])[0] for it in timed})
    dk = {c: torch.zeros(att.kv_shape(), device=dev) for c in own_kv}
    dv = {c: torch.zeros(att.kv_shape(), device=dev) for c in own_kv}

    def step():
        if w.backward:
            for a in owners:
                dq[a].zero_()
            for c in own_kv:
                dk[c].zero_()
                dv[c].zero_()
        att.forward_items(timed, q, k, v, partials)
        for a in owners:
            att.merge_owner(a, partials, o[a], lse[a])
        if w.backward:
            att.backward_items(timed, q, k, v, o, lse, d_o, delta, dq, dk, dv)

    per_pair = w.batch * w.heads_q * w.head_dim
    n_pairs = sum(visible_pairs(it, w.chunk, w.window, w.n_global) for it in timed)
    fwd_flop = n_pairs * per_pair * 4
    bwd_flop = n_pairs * per_pair * 10 if w.backward else 0
    flop = fwd_flop + bwd_flop

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else \
        0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    tflops = flop / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # Per-launch timing of the two compute calls (HIP events on the stream the
    # library launches on: torch's current stream).
    stream = torch.cuda.current_stream()

    def per_call(fn, items):
        evs = []
        for it in items:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(it)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs)

    def fwd_call(it):
        a, kc = it[2], it[3]
        o_part, l_part = partials[(a, kc)]
        for d, bs, src, rs in att.calls(a, kc):
            dfa.dfa_attn_fwd_partial(d, q[a][bs], k[src][bs, rs], v[src][bs, rs], o_part[bs],
                                     l_part[bs], None, att.workspace(d, dfa.DFA_OP_FWD))

    def bwd_call(part):
        def call(it):
            a, kc = it[2], it[3]
            for d, bs, src, rs in att.calls(a, kc):
                dfa.dfa_test_bwd_part(d, q[a][bs], k[src][bs, rs], v[src][bs, rs], lse[a][bs],
                                      d_o[a][bs], delta[a][bs], dq[a][bs], dk[src][bs, rs],
                                      dv[src][bs, rs], part, None,
                                      att.workspace(d, dfa.DFA_OP_BWD))
        return call

    pairs_x_heads = n_pairs * w.batch * w.heads_q
    # name in the profiler -> (time per step, algorithmic FLOP per step,
    # executed MFMA FLOP per step).  Algorithmic: each kernel's share of the
    # method's work, so that the shares sum to the 14d per visible pair the
    # step counts (forward 4d: S, PV; dK/dV 8d: S, dP, dV, dK; dQ 2d: the dQ
    # product; its S and dP repeat the dK/dV kernel's and are executed work
    # only, 4d more).
    names = KERNEL_NAMES if w.dtype == "bf16" else KERNEL_NAMES_F32
    calls = [d for it in timed for d, *_ in att.calls(it[2], it[3])]
    # Kernel launches per step: one forward kernel per call; the dK/dV kernel
    # runs a diagonal pair of whole key blocks as two or three row-band
    # launches, so per-launch figures divide by the library's own count.
    kernels = {names["fwd"]: (per_call(fwd_call, timed), pairs_x_heads * 4 * w.head_dim,
                              pairs_x_heads * 4 * w.head_dim, len(calls))}
    if w.backward:
        kernels[names["dkdv"]] = (per_call(bwd_call(1), timed), pairs_x_heads * 8 * w.head_dim,
                                  pairs_x_heads * 8 * w.head_dim,
                                  sum(dfa.dfa_test_bwd_launches(d, 1) for d in calls))
        kernels[names["dq"]] = (per_call(bwd_call(2), timed), pairs_x_heads * 2 * w.head_dim,
                                pairs_x_heads * 6 * w.head_dim,
                                sum(dfa.dfa_test_bwd_launches(d, 2) for d in calls))
    nl = len(timed)
    name, (kms, kflop, _, kl) = max(kernels.items(), key=lambda kv: kv[1][0])
    achieved = kflop / (kms * 1e-3) / 1e12
    tf = lambda f, ms: round(f / (ms * 1e-3) / 1e12, 2)  # noqa: E731
    tdetail = traffic_of(name, kl, w.name)
    roofline = {"bound": "mfma" if w.dtype == "bf16" else "alu", "kernel": name, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if tdetail is None else tdetail["bytes_per_launch"],
                "traffic_detail": tdetail, "avg_launch_ms": round(kms / kl, 3),
                "launches_per_step": kl, "flop_per_launch": kflop / kl,
                "others": {n: {"avg_launch_ms": round(x[0] / x[3], 3), "launches_per_step": x[3],
                               "tflops": tf(x[1], x[0]), "executed_tflops": tf(x[2], x[0])}
                           for n, x in kernels.items()}}
    if w.backward:
        bms = kernels[names["dkdv"]][0] + kernels[names["dq"]][0]
        roofline["backward_pair"] = {"avg_pair_ms": round(bms / nl, 3),
                                     "tflops": tf(pairs_x_heads * 10 * w.head_dim, bms),
                                     "executed_tflops": tf(pairs_x_heads * 14 * w.head_dim, bms)}

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ARITH_DTYPE[w.dtype], "data": "synthetic",
        "pct_of_peak": round(100 * tflops / peak, 2),
        "median_ms_per_step": round(median_ms, 3),
        "median_value": round(flop / (median_ms * 1e-3) / 1e12, 2),
        "config": {"workload": w.name, "chunk": w.chunk, "workers": w.workers,
                   "total_seq": w.total_len, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "batch": w.batch,
                   "share": (f"worker {w.share_of} of {w.workers}" if w.share_of >= 0
                             else "all pairs"),
                   "pairs_timed": len(timed), "backward": w.backward, "window": w.window,
                   "n_global": w.n_global,
                   "algorithmic_flop_per_step": flop, "wall_s_timed": round(wall, 3),
                   "reference_copy_bytes": REFERENCE_COPY_BYTES,
                   "input_gen_s": round(gen_s, 1)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        del q, k, v, d_o, partials, o, lse, delta, dq, dk, dv
        torch.cuda.empty_cache()
        a = w.share_of if w.share_of >= 0 else w.workers - 1
        kv_lo = min(it[3] for it in att.items_of_owner(a) if it[3] >= 0)
        result["cpu_baseline"] = cpu_baseline(w, host, w.share_of, args.cpu_seconds, kv_lo)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
