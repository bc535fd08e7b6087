"""Host orchestration of the chunked causal attention on one GPU.

P virtual workers hold P contiguous chunks of C tokens ([DistFlashAttn
§3.1]).  The schedule (from libdfa's dfa_balanced_schedule, or
dfa_window_schedule for a local sliding window, App. F) lists the
(query chunk, key/value chunk) pairs; each pair is one dfa_attn_fwd_partial
call, an owner's partials are combined by dfa_lse_merge in ascending
key/value chunk order, and the backward replays the owner's pairs through
dfa_attn_bwd from the merged O and LSE.  On one GPU the workers are plain
work items on one stream; a helper's returned (O, LSE) is simply a buffer
the owner's merge reads.

This module only sequences library calls; every number is computed by the
library's kernels.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import dfa

_TD = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class ChunkedCausalAttention:
    workers: int
    chunk: int
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str = "bf16"
    balanced: bool = True
    scale: float | None = None
    window: int = 0  # 0: full causal attention; > 0: local sliding window of that many tokens

    def __post_init__(self):
        if self.window > 0:
            self.items, self.num_steps = dfa.dfa_window_schedule(self.workers, self.chunk,
                                                                 self.window)
        else:
            self.items, self.num_steps = dfa.dfa_balanced_schedule(self.workers, self.balanced)
        if self.scale is None:
            self.scale = self.head_dim ** -0.5

    # ---- schedule views -------------------------------------------------
    def items_of_worker(self, w: int):
        return [it for it in self.items if it[1] == w]

    def items_of_owner(self, a: int):
        """Every pair whose query rows belong to chunk a, ascending kv chunk."""
        return sorted((it for it in self.items if it[5] == a), key=lambda it: it[3])

    def desc(self, q_chunk: int, kv_chunk: int) -> dfa.AttnDesc:
        c = self.chunk
        return dfa.make_desc(self.batch, self.heads_q, self.heads_kv, self.head_dim, c, c,
                             q_chunk * c, kv_chunk * c, True, self.scale, self.dtype, self.window)

    # ---- buffers --------------------------------------------------------
    def q_shape(self):
        return (self.batch, self.chunk, self.heads_q, self.head_dim)

    def kv_shape(self):
        return (self.batch, self.chunk, self.heads_kv, self.head_dim)

    def lse_shape(self):
        return (self.batch, self.heads_q, self.chunk)

    def new_partial(self, device="cuda"):
        return (torch.empty(self.q_shape(), dtype=torch.float32, device=device),
                torch.empty(self.lse_shape(), dtype=torch.float32, device=device))

    # ---- the hot path -----------------------------------------------------
    def forward_items(self, items, q, k, v, partials, stream=None):
        """q, k, v: chunk index -> tensor; partials: (a, c) -> (o_part, lse)."""
        for it in items:
            a, c = it[2], it[3]
            o_part, lse = partials[(a, c)]
            dfa.dfa_attn_fwd_partial(self.desc(a, c), q[a], k[c], v[c], o_part, lse, stream)

    def merge_owner(self, a, partials, o_out, lse_out, stream=None):
        its = self.items_of_owner(a)
        dfa.dfa_lse_merge([partials[(a, it[3])][0] for it in its],
                          [partials[(a, it[3])][1] for it in its],
                          self.batch, self.heads_q, self.chunk, self.head_dim, self.dtype,
                          o_out, lse_out, stream)

    def backward_items(self, items, q, k, v, o, lse, d_o, delta, dq, dk, dv, have_delta=None,
                       stream=None):
        """Adds each pair's dQ / dK / dV into dq[a], dk[c], dv[c] (caller-zeroed).

        o, lse, d_o, delta: query chunk -> tensors (final O and LSE).  The
        delta of a query chunk is computed on its first pair here and reused
        (have_delta tracks which chunks already hold it)."""
        have = set() if have_delta is None else have_delta
        for it in items:
            a, c = it[2], it[3]
            first = a not in have
            dfa.dfa_attn_bwd(self.desc(a, c), q[a], k[c], v[c], o[a] if first else None, lse[a],
                             d_o[a], delta[a], first, dq[a], dk[c], dv[c], stream)
            have.add(a)
        return have
