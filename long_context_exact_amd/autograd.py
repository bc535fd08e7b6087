"""torch.autograd binding of the chunked causal attention.

`chunked_attention(q, k, v, att)` runs the whole sequence through the
library: every pair of the schedule (`dfa_attn_fwd_partial`), every owner's
LSE merge (`dfa_lse_merge`), and on backward every pair's
`dfa_attn_bwd` from the saved final O and LSE.  The backward never runs the
attention forward again ([DistFlashAttn §3.3]: the attention backward only
needs the attention output and its statistics).

Tensors are [B, N, H, d] with N = workers * chunk, in the runner's dtype.
This module only moves tensors and sequences library calls.
"""

from __future__ import annotations

import torch

from .runner import ChunkedCausalAttention

_TD = {"f32": torch.float32, "bf16": torch.bfloat16}

# Number of attention forward passes run so far (the forward of
# `chunked_attention`, never its backward): lets callers check where a
# checkpointing strategy recomputes attention.
FORWARD_CALLS = [0]


def _chunks(x: torch.Tensor, c: int, p: int):
    """Per-chunk contiguous views (copies only when B > 1 makes them strided)."""
    return {a: x[:, a * c:(a + 1) * c].contiguous() for a in range(p)}


def attention_forward(att: ChunkedCausalAttention, q, k, v):
    """(o [B, N, Hq, d] in the input dtype, lse {chunk: [B, Hq, C] fp32})."""
    FORWARD_CALLS[0] += 1
    p, c = att.workers, att.chunk
    qc, kc, vc = _chunks(q, c, p), _chunks(k, c, p), _chunks(v, c, p)
    o = torch.empty_like(q)
    lse = {a: torch.empty(att.lse_shape(), dtype=torch.float32, device=q.device)
           for a in range(p)}
    for a in range(p):
        its = att.items_of_owner(a)
        parts = {(it[2], it[3]): att.new_partial(q.device) for it in its}
        att.forward_items(its, qc, kc, vc, parts)
        o_a = torch.empty(att.q_shape(), dtype=q.dtype, device=q.device)
        att.merge_owner(a, parts, o_a, lse[a])
        o[:, a * c:(a + 1) * c] = o_a
        del parts
    return o, lse


def attention_backward(att: ChunkedCausalAttention, q, k, v, o, lse, d_o):
    """(dq, dk, dv) in the input dtype, from the saved final O and LSE."""
    p, c = att.workers, att.chunk
    qc, kc, vc = _chunks(q, c, p), _chunks(k, c, p), _chunks(v, c, p)
    oc, doc = _chunks(o, c, p), _chunks(d_o.to(q.dtype), c, p)
    dq = {a: torch.zeros(att.q_shape(), dtype=torch.float32, device=q.device) for a in range(p)}
    dk = {a: torch.zeros(att.kv_shape(), dtype=torch.float32, device=q.device) for a in range(p)}
    dv = {a: torch.zeros(att.kv_shape(), dtype=torch.float32, device=q.device) for a in range(p)}
    delta = {a: torch.empty(att.lse_shape(), dtype=torch.float32, device=q.device)
             for a in range(p)}
    att.backward_items(att.items, qc, kc, vc, oc, lse, doc, delta, dq, dk, dv)
    cat = lambda d: torch.cat([d[a] for a in range(p)], dim=1).to(q.dtype)  # noqa: E731
    return cat(dq), cat(dk), cat(dv)


class ChunkedAttentionFn(torch.autograd.Function):
    """Autograd node: forward = schedule + merges, backward = per-pair
    backward from the saved O and LSE (no attention forward in backward)."""

    @staticmethod
    def forward(ctx, q, k, v, att):
        o, lse = attention_forward(att, q, k, v)
        ctx.att = att
        ctx.lse = lse
        ctx.save_for_backward(q, k, v, o)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o = ctx.saved_tensors
        dq, dk, dv = attention_backward(ctx.att, q, k, v, o, ctx.lse, d_o.contiguous())
        return dq, dk, dv, None


def chunked_attention(q, k, v, att: ChunkedCausalAttention):
    return ChunkedAttentionFn.apply(q, k, v, att)
