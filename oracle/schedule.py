"""Chunk-pair schedules and the causal tile map — TEST INFRASTRUCTURE ONLY.

A sequence of N tokens is cut into P contiguous equal chunks, worker w
holding chunk w ([DistFlashAttn §3.1]).  Causal attention needs the pair
(query chunk a, key/value chunk c) only when a >= c; (a, a) is the diagonal
pair and needs the element mask, every a > c pair is full.

Unbalanced schedule ([DistFlashAttn §3.2]; App. B, Fig. 5): at step t,
worker w >= t computes its own queries against chunk w - t, the others
idle.  P steps; about half the workers idle.

Load-balanced schedule ([DistFlashAttn §1, its token-level balancing;
§3.2 and Fig. 3; App. B, Fig. 6]).  The figure itself is not in
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

Local sliding window ([DistFlashAttn App. F, discussion of sparse
attention]): when a query sees only the W tokens ending at itself, the work
is already nearly even across workers, so each worker keeps its own query
chunk and only shortens the loop of the unbalanced schedule to the key/value
chunks that hold keys inside some window of its queries (with W <= C worker
7 of 8 visits chunks 6 and 7 only).  No helpers, no rebalancing.

Items are tuples (step, worker, q_chunk, kv_chunk, kind, owner), sorted by
(step, worker); kind 0 = diagonal (causal mask), 1 = full, 2 = band (an
off-diagonal pair that a sliding window cuts: some pairs of it hidden);
owner = q_chunk.
"""

from __future__ import annotations

import numpy as np

__all__ = ["balanced_schedule", "unbalanced_schedule", "window_schedule",
           "global_window_schedule", "causal_tile_map", "DIAG", "FULL", "BAND", "GLOBAL"]

DIAG = 0
FULL = 1
BAND = 2
GLOBAL = 3


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


def window_schedule(num_workers: int, chunk_len: int, window: int):
    """(items, num_steps) of the sliding-window schedule: worker w does
    (w, w - t) at step t for every t whose chunk pair holds a pair of
    tokens less than `window` apart (the closest such pair is (t - 1) * C + 1
    positions apart for t >= 1); kind FULL when even the farthest pair,
    (t + 1) * C - 1 apart, is inside the window, else BAND."""
    p, c, w_ = int(num_workers), int(chunk_len), int(window)
    if p < 1 or c < 1 or w_ < 1:
        raise ValueError("num_workers, chunk_len and window must be >= 1")
    items = []
    t = 0
    while t < p and (t == 0 or (t - 1) * c + 1 < w_):
        kind = DIAG if t == 0 else (FULL if (t + 1) * c - 1 < w_ else BAND)
        for w in range(t, p):
            items.append((t, w, w, w - t, kind, w))
        t += 1
    return items, t


def global_window_schedule(num_workers: int, chunk_len: int, window: int, n_global: int):
    """(items, num_steps) of a sliding window plus G = n_global global tokens
    replicated on every worker ([App. F]: global tokens may be replicated so
    that no step gathers them).  The global tokens are the first G positions
    (G <= C, all in chunk 0).  Every worker w first does its global item
    (step 0, kv chunk -1, kind GLOBAL): its queries against the G global
    keys, from its own replica.  Its window items are those of
    ``window_schedule``, except that a pair over chunk 0 covers only keys
    G..C-1 (keys below G belong to the global item, so none is counted
    twice) and is dropped when G = C.  Sorted by (step, worker, kv chunk)."""
    p, c, w_, g = int(num_workers), int(chunk_len), int(window), int(n_global)
    if g < 1 or g > c:
        raise ValueError("n_global must be in [1, chunk_len]")
    items, steps = window_schedule(p, c, w_)
    items = [it for it in items if not (it[3] == 0 and g == c)]
    items += [(0, w, w, -1, GLOBAL, w) for w in range(p)]
    items.sort(key=lambda it: (it[0], it[1], it[3]))
    return items, steps


def causal_tile_map(len_q: int, len_k: int, q_start: int, kv_start: int,
                    causal: bool, bm: int, bn: int, window: int = 0) -> np.ndarray:
    """Which (query tile, key tile) pairs of one chunk pair carry visible
    scores, and which of them straddle the causal diagonal.

    Tile (qt, kt) covers query rows [qt*bm, min((qt+1)*bm, len_q)) and key
    columns [kt*bn, min((kt+1)*bn, len_k)).  With global positions the tile
    holds a visible score iff its first key is not after its last query:
        kv_start + kt*bn <= q_start + min((qt+1)*bm, len_q) - 1,
    and needs the element mask iff, in addition, its last key is after its
    first query.  Skipping the other tiles is how causal attention avoids the
    doubled work the paper attributes to Ring Attention (§2).  With a sliding
    window of W tokens a tile is also skipped when its last key is W or more
    positions behind its first query, and masked when its first key is W or
    more positions behind its last query (App. F).

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
            elif first_k <= last_q and (window <= 0 or first_q - last_k < window):
                masked = last_k > first_q or (window > 0 and last_q - first_k >= window)
                out[qt, kt] = 2 if masked else 1
    return out
