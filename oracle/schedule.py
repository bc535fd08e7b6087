"""Chunk-pair schedules and the causal tile map — TEST INFRASTRUCTURE ONLY.

A sequence of N tokens is cut into P contiguous equal chunks, worker w
holding chunk w ([DistFlashAttn §3.1]).  Causal attention needs the pair
(query chunk a, key/value chunk c) only when a >= c; (a, a) is the diagonal
pair and needs the element mask, every a > c pair is full.

Unbalanced schedule ([DistFlashAttn §3.2]; App. B, Fig. 5): at step t,
worker w >= t computes its own queries against chunk w - t, the others
idle.  P steps; about half the workers idle.

Load-balanced schedule ([DistFlashAttn §1 "token-level workload
balancing", §3.2 and Fig. 3; App. B, Fig. 6]).  The figure itself is not in
the text, so the assignment is the plainest one that the stated facts fix:
  * step 0: every worker does its diagonal pair (w, w);
  * step t = 1 .. floor(P/2): worker w >= t does (w, w - t) for itself;
    worker h < t, which the unbalanced schedule leaves idle, helps the
    heaviest worker h + P - t with the pair (h + P - t, h), i.e. against the
    helper's own key/value chunk, and returns (O, LSE) to that owner —
    unless P - t == t, where that pair would repeat one already done.
It reproduces the paper's theoretical speedups over one device at P = 8
(7.2x balanced, 4.5x unbalanced; §4.5, Fig. 4), the idle fraction that
tends to zero for even P (§3.2), the doubling over the unbalanced version
(§1) and a forward traffic of N*d elements per worker (App. D).

Items are tuples (step, worker, q_chunk, kv_chunk, kind, owner), sorted by
(step, worker); kind 0 = diagonal (causal mask), 1 = full; owner = q_chunk.
"""

from __future__ import annotations

import numpy as np

__all__ = ["balanced_schedule", "unbalanced_schedule", "causal_tile_map",
           "DIAG", "FULL"]

DIAG = 0
FULL = 1


def unbalanced_schedule(num_workers: int):
    """(items, num_steps) of the unbalanced causal ring schedule."""
    p = int(num_workers)
    if p < 1:
        raise ValueError("num_workers must be >= 1")
    items = []
    for t in range(p):
        for w in range(p):
            if w >= t:
                items.append((t, w, w, w - t, DIAG if t == 0 else FULL, w))
    return items, p


def balanced_schedule(num_workers: int):
    """(items, num_steps) of the token-level load-balanced schedule."""
    p = int(num_workers)
    if p < 1:
        raise ValueError("num_workers must be >= 1")
    items = []
    steps = 1 + p // 2
    for t in range(steps):
        for w in range(p):
            if t == 0:
                items.append((0, w, w, w, DIAG, w))
            elif w >= t:
                items.append((t, w, w, w - t, FULL, w))
            elif p - t > t:
                owner = w + p - t
                items.append((t, w, owner, w, FULL, owner))
    return items, steps


def causal_tile_map(len_q: int, len_k: int, q_start: int, kv_start: int,
                    causal: bool, bm: int, bn: int) -> np.ndarray:
    """Which (query tile, key tile) pairs of one chunk pair carry visible
    scores, and which of them straddle the causal diagonal.

    Tile (qt, kt) covers query rows [qt*bm, min((qt+1)*bm, len_q)) and key
    columns [kt*bn, min((kt+1)*bn, len_k)).  With global positions the tile
    holds a visible score iff its first key is not after its last query:
        kv_start + kt*bn <= q_start + min((qt+1)*bm, len_q) - 1,
    and needs the element mask iff, in addition, its last key is after its
    first query.  Skipping the other tiles is how causal attention avoids the
    doubled work the paper attributes to Ring Attention (§2).

    Returns uint8 [ceil(len_q/bm), ceil(len_k/bn)]: 0 skipped, 1 visited
    unmasked, 2 visited with the element mask.
    """
    nqt = -(-len_q // bm)
    nkt = -(-len_k // bn)
    out = np.zeros((nqt, nkt), dtype=np.uint8)
    for qt in range(nqt):
        first_q = q_start + qt * bm
        last_q = q_start + min((qt + 1) * bm, len_q) - 1
        for kt in range(nkt):
            first_k = kv_start + kt * bn
            last_k = kv_start + min((kt + 1) * bn, len_k) - 1
            if not causal:
                out[qt, kt] = 1
            elif first_k <= last_q:
                out[qt, kt] = 2 if last_k > first_q else 1
    return out
