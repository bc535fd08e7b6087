"""Exact causal softmax attention in float64 — TEST INFRASTRUCTURE ONLY.

The paper computes *exact* attention (abstract; App. F names exact attention
as its scope) and its rematerialisation-aware checkpointing leaves every
number unchanged (§1, §2).  So the oracle is the
plain definition written out: every query row takes one full softmax over
all of its visible keys at once.  There is no online rescaling, no tiling
and no chunk merge in ``attention_fwd``; query rows are walked in blocks only
to bound memory.  A matrix product (numpy, float64) is the one library step.

Notation (one head h of one batch row b):
    sigma      the softmax scale (1/sqrt(d) in every workload)
    G          Hq / Hkv, query heads per key/value head; g(h) = h // G
    q0, k0     global token index of row 0 of the query / key chunk
    J(i)       visible keys of query i: {j : k0 + j <= q0 + i} when causal;
               with a sliding window of W tokens also q0 + i - (k0 + j) < W
               (a query sees itself and the W - 1 tokens before it); with
               n_global = G > 0 global tokens, keys at positions < G are
               visible through the window as well (each still counted once)
    s_ij       sigma * <Q_i, K_j>
    LSE_i      natural-log log-sum-exp of s_ij over J(i)   (-inf if J(i) empty)
    P_ij       exp(s_ij - LSE_i) on J(i), 0 elsewhere
    O_i        sum_j P_ij V_j                              (0 if J(i) empty)

Layouts follow the boundary: Q, O, dO, dQ [B, Lq, Hq, d]; K, V, dK, dV
[B, Lk, Hkv, d]; LSE and D [B, Hq, Lq].
"""

from __future__ import annotations

import numpy as np

__all__ = ["attention_fwd", "lse_merge", "attention_bwd", "attention_delta"]

# Rows per block: keeps one [rows, Lk] float64 score block near 128 MiB.
_BLOCK_ELEMS = 1 << 24


def _rows_per_block(lk: int) -> int:
    return int(max(1, min(512, _BLOCK_ELEMS // max(lk, 1))))


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, L, H, d]")
    b, lq, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    hkv = k.shape[2]
    if hkv == 0 or hq % hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return b, lq, hq, k.shape[1], hkv, d


def _check_window(causal: bool, window: int, n_global: int = 0):
    window, n_global = int(window), int(n_global)
    if window < 0 or n_global < 0:
        raise ValueError("window and n_global must be >= 0")
    if (window > 0 or n_global > 0) and not causal:
        raise ValueError("a sliding window or global tokens apply to causal attention only")
    return window, n_global


def _visible(rows: np.ndarray, lk: int, q0: int, k0: int, causal: bool, window: int = 0,
             n_global: int = 0):
    """Boolean [len(rows), lk]: key j visible to query i (global positions,
    inclusive diagonal: a query sees itself and every earlier token; §3.2:
    a worker attends over the prefix up to its own chunk and nothing later).  window > 0 keeps only
    the keys less than `window` positions behind the query: the local
    sliding window of [App. F], which lets a worker skip non-local keys.
    n_global = G > 0 adds back the global tokens of App. F's global
    attention, read as the first G positions of the sequence: a query also
    sees every global token at or before it."""
    if not causal:
        return np.ones((rows.size, lk), dtype=bool)
    kpos = k0 + np.arange(lk)[None, :]
    dist = (q0 + rows[:, None]) - kpos
    vis = dist >= 0
    if window > 0:
        vis &= (dist < window) | (kpos < n_global)
    return vis


def attention_fwd(q, k, v, scale, causal=True, q_start=0, kv_start=0, window=0, n_global=0):
    """Exact attention output and LSE for one (query chunk, key/value chunk)
    block, or for a whole sequence (q_start = kv_start = 0).

    The partial state a worker returns for a chunk pair is the normalised
    output plus its log-sum-exp ([DistFlashAttn App. D]: per pair the
    forward produces the output together with its log-sum-exp; §3.2: a helper
    sends that state back to the owner, which rescales and combines it).

    Returns (o [B,Lq,Hq,d] float64, lse [B,Hq,Lq] float64).  Rows that see
    no key get o = 0 and lse = -inf.  window > 0 (causal only): the local
    sliding window described in [App. F]; n_global > 0 (with a window): the
    first n_global positions are global tokens every later query sees.
    """
    window, n_global = _check_window(causal, window, n_global)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, lq, hq, lk, hkv, d = _check_shapes(q, k, v)
    group = hq // hkv
    o = np.zeros((b, lq, hq, d), dtype=np.float64)
    lse = np.full((b, hq, lq), -np.inf, dtype=np.float64)
    if lq == 0 or lk == 0:
        return o, lse
    rb = _rows_per_block(lk)
    for bi in range(b):
        for h in range(hq):
            kg = k[bi, :, h // group, :]          # [Lk, d]
            vg = v[bi, :, h // group, :]
            for r0 in range(0, lq, rb):
                rows = np.arange(r0, min(lq, r0 + rb))
                s = scale * (q[bi, rows, h, :] @ kg.T)          # [R, Lk]
                vis = _visible(rows, lk, q_start, kv_start, causal, window, n_global)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)                                # -inf if empty
                live = np.isfinite(m)
                if not live.any():
                    continue
                sl, ml = s[live], m[live]
                row_lse = ml + np.log(np.exp(sl - ml[:, None]).sum(axis=1))
                p = np.exp(sl - row_lse[:, None])                # masked -> 0
                lse[bi, h, rows[live]] = row_lse
                o[bi, rows[live], h, :] = p @ vg
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Combine partial states of the same query rows over disjoint key sets
    ([DistFlashAttn §3.2, Fig. 3]: the owner rescales the partial outputs it
    receives using their softmax statistics).

    With LSE^(r) the natural-log log-sum-exp over key set r, the union's
    LSE is logsumexp_r LSE^(r), and each normalised partial is reweighted by
    its share exp(LSE^(r) - LSE) of the union's softmax mass.  Rows whose
    every partial is empty (-inf) stay o = 0, lse = -inf.

    o_parts: sequence of [B, Lq, H, d]; lse_parts: sequence of [B, H, Lq].
    Returns (o, lse) in float64.
    """
    if len(o_parts) == 0 or len(o_parts) != len(lse_parts):
        raise ValueError("need the same positive number of O and LSE parts")
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])  # [n,B,H,Lq]
    m = lses.max(axis=0)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    total = np.exp(lses - m_safe[None]).sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, m_safe + np.log(total), -np.inf)
    lse_safe = np.where(live, lse, 0.0)
    o = np.zeros(np.asarray(o_parts[0]).shape, dtype=np.float64)
    for o_r, lse_r in zip(o_parts, lses):
        w = np.where(live, np.exp(lse_r - lse_safe), 0.0)        # [B, H, Lq]
        o += np.transpose(w, (0, 2, 1))[..., None] * np.asarray(o_r, dtype=np.float64)
    return o, lse


def attention_delta(o, do):
    """D_i = <dO_i, O_i> per (batch, head, row), from the final output.
    Returns [B, Hq, Lq] float64."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.transpose((o * do).sum(axis=3), (0, 2, 1))


def attention_bwd(q, k, v, o, lse, do, scale, causal=True, q_start=0,
                  kv_start=0, delta=None, window=0, n_global=0):
    """Gradients of L = sum_{i,h} <dO_i, O_i> restricted to one block of
    (query rows, key columns), from the *saved* final O and LSE.

    The backward never re-runs the forward: it consumes the checkpointed
    attention output and its statistics ([DistFlashAttn §3.3]: checkpointing
    the FlashAttention output lets the attention backward reuse it, so the
    forward runs once).  With P from the final LSE and D from the final O,
        dP_ij = <dO_i, V_j>,  dS_ij = P_ij (dP_ij - D_i),
        dQ_i  = sigma * sum_j dS_ij K_j,
        dK_j  = sigma * sum_{h in group} sum_i dS_ij Q_i,
        dV_j  = sum_{h in group} sum_i P_ij dO_i.
    These sums are linear in the block, so adding the results over every
    block of a sequence gives the whole-sequence gradient.

    o, do: [B,Lq,Hq,d]; lse: [B,Hq,Lq] (final, merged); delta: optional
    [B,Hq,Lq] (computed from o and do when None); window and n_global as
    in ``attention_fwd``.
    Returns (dq [B,Lq,Hq,d], dk [B,Lk,Hkv,d], dv [B,Lk,Hkv,d]) in float64.
    """
    window, n_global = _check_window(causal, window, n_global)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    b, lq, hq, lk, hkv, d = _check_shapes(q, k, v)
    group = hq // hkv
    if delta is None:
        delta = attention_delta(o, do)
    delta = np.asarray(delta, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if lq == 0 or lk == 0:
        return dq, dk, dv
    rb = _rows_per_block(lk)
    for bi in range(b):
        for h in range(hq):
            g = h // group
            kg, vg = k[bi, :, g, :], v[bi, :, g, :]
            for r0 in range(0, lq, rb):
                rows = np.arange(r0, min(lq, r0 + rb))
                row_lse = lse[bi, h, rows]
                live = np.isfinite(row_lse)
                if not live.any():
                    continue
                rows, row_lse = rows[live], row_lse[live]
                qi, doi = q[bi, rows, h, :], do[bi, rows, h, :]
                s = scale * (qi @ kg.T)
                vis = _visible(rows, lk, q_start, kv_start, causal, window, n_global)
                p = np.where(vis, np.exp(np.where(vis, s, 0.0) - row_lse[:, None]), 0.0)
                dp = doi @ vg.T
                ds = p * (dp - delta[bi, h, rows][:, None])
                dq[bi, rows, h, :] += scale * (ds @ kg)
                dk[bi, :, g, :] += scale * (ds.T @ qi)
                dv[bi, :, g, :] += p.T @ doi
    return dq, dk, dv
