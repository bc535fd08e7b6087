"""Host orchestration of the chunked causal attention on one GPU.

P virtual workers hold P contiguous chunks of C tokens ([DistFlashAttn
§3.1]).  The schedule (from libdfa's dfa_balanced_schedule, dfa_window_schedule
for a local sliding window, or dfa_global_window_schedule for a window plus
replicated global tokens, App. F) lists the (query chunk, key/value chunk)
pairs; each pair is one dfa_attn_fwd_partial call, an owner's partials are
combined by dfa_lse_merge in ascending key/value chunk order, and the
backward replays the owner's pairs through dfa_attn_bwd from the merged O
and LSE.

With G global tokens (the first G positions, in chunk 0) a global item
(kv chunk -1) reads keys 0..G-1 and a pair over chunk 0 reads keys G..C-1.
Those key ranges are row ranges of chunk 0's tensors; the kernels take
[B, len, H, d] contiguous tensors, so with B > 1 such a pair runs as one
call per batch row (each a contiguous slice).  Every worker reads the same
global rows: on one GPU the replicas the pages describe are one tensor,
and their gradients (summed over workers by an all-reduce on many GPUs)
add into the same dK/dV rows.  On one GPU the workers are plain
work items on one stream; a helper's returned (O, LSE) is simply a buffer
the owner's merge reads.

The scratch the kernels need (the forward's transposed V, the backward's
row-split partials) is a workspace per device and stream that this object
owns: a torch tensor grown to the largest size any call on that stream has
asked for, passed to every call.  Calls on one stream are ordered, so they
may share it; calls on different streams get different workspaces and may
overlap.  The library itself allocates nothing.

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
    n_global: int = 0  # > 0 (with a window): the first n_global tokens are global

    def __post_init__(self):
        if self.n_global > 0:
            if self.window <= 0:
                raise ValueError("global tokens need a sliding window (else every key is visible)")
            self.items, self.num_steps = dfa.dfa_global_window_schedule(
                self.workers, self.chunk, self.window, self.n_global)
        elif self.window > 0:
            self.items, self.num_steps = dfa.dfa_window_schedule(self.workers, self.chunk,
                                                                 self.window)
        else:
            self.items, self.num_steps = dfa.dfa_balanced_schedule(self.workers, self.balanced)
        if self.scale is None:
            self.scale = self.head_dim ** -0.5
        self._ws = {}

    def workspace(self, desc: dfa.AttnDesc, op: int, device=None, stream=None):
        """This object's workspace for calls on `stream` (None: the current
        stream) of `device`, grown to what `desc` needs for `op`
        (dfa.DFA_OP_FWD / DFA_OP_BWD).  It is allocated on that stream, so
        when growing drops the old tensor torch reuses its memory only for
        work queued after the calls already on that stream."""
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else \
            torch.device(device)
        ts = dfa._torch_stream(stream)
        key = (dev, ts.cuda_stream)
        need = dfa.dfa_attn_workspace_size(desc, op)
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            with torch.cuda.stream(ts):
                ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            self._ws[key] = ws
        return ws

    # ---- schedule views -------------------------------------------------
    def items_of_worker(self, w: int):
        return [it for it in self.items if it[1] == w]

    def items_of_owner(self, a: int):
        """Every pair whose query rows belong to chunk a, ascending kv chunk."""
        return sorted((it for it in self.items if it[5] == a), key=lambda it: it[3])

    def desc(self, q_chunk: int, kv_chunk: int) -> dfa.AttnDesc:
        """Descriptor of a pair over whole chunks (no global tokens involved)."""
        c = self.chunk
        return dfa.make_desc(self.batch, self.heads_q, self.heads_kv, self.head_dim, c, c,
                             q_chunk * c, kv_chunk * c, True, self.scale, self.dtype, self.window)

    def kv_rows(self, kv_chunk: int):
        """(source chunk, first row, end row, kv_start, window) of an item's keys."""
        c, g = self.chunk, self.n_global
        if kv_chunk == -1:            # global item: keys 0..G-1, causal, no window
            return 0, 0, g, 0, 0
        if kv_chunk == 0 and g > 0:   # chunk 0 past its global prefix
            return 0, g, c, g, self.window
        return kv_chunk, 0, c, kv_chunk * c, self.window

    def calls(self, q_chunk: int, kv_chunk: int):
        """The library calls of one item: (desc, batch slice, source chunk,
        row slice); one call over every batch row unless the keys are a
        sub-range of the chunk and B > 1."""
        src, r0, r1, k0, win = self.kv_rows(kv_chunk)
        c = self.chunk
        if (r0 == 0 and r1 == c) or self.batch == 1:
            parts = [(slice(None), self.batch)]
        else:
            parts = [(slice(b, b + 1), 1) for b in range(self.batch)]
        for bs, nb in parts:
            d = dfa.make_desc(nb, self.heads_q, self.heads_kv, self.head_dim, c, r1 - r0,
                              q_chunk * c, k0, True, self.scale, self.dtype, win)
            yield d, bs, src, slice(r0, r1)

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
            for d, bs, src, rs in self.calls(a, c):
                dfa.dfa_attn_fwd_partial(d, q[a][bs], k[src][bs, rs], v[src][bs, rs], o_part[bs],
                                         lse[bs], stream,
                                         self.workspace(d, dfa.DFA_OP_FWD, q[a].device, stream))

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
        (have_delta tracks which (chunk, batch row) pairs already hold it)."""
        have = set() if have_delta is None else have_delta
        for it in items:
            a, c = it[2], it[3]
            for d, bs, src, rs in self.calls(a, c):
                rows = range(self.batch) if bs.start is None else [bs.start]
                first = (a, rows[0]) not in have
                assert all(((a, b) not in have) == first for b in rows)
                dfa.dfa_attn_bwd(d, q[a][bs], k[src][bs, rs], v[src][bs, rs],
                                 o[a][bs] if first else None, lse[a][bs], d_o[a][bs],
                                 delta[a][bs], first, dq[a][bs], dk[src][bs, rs],
                                 dv[src][bs, rs], stream,
                                 self.workspace(d, dfa.DFA_OP_BWD, q[a].device, stream))
                have.update((a, b) for b in rows)
        return have

    # ---- communication / computation overlap (one GPU, two streams) -------
    def forward_worker_overlapped(self, w, q, k, v, partials, overlap=True):
        """Worker w's forward items in step order with the per-step exchange
        emulated on a second stream ([DistFlashAttn §3.2]: the next block's
        key/value tensors are prefetched while the current block computes, on
        separate streams; §1, Fig. 2).

        An owner item (w, c), c != w, needs chunk c's K and V from worker c;
        a helper item (a, w) needs owner a's Q and sends its (O, LSE) back.
        Each received tensor lands in one of two receive slots by a
        DMA-engine copy (dfa_chunk_transfer: no compute units, as a link
        transfer) on the communication stream; the copy for step t + 1 is
        issued before step t computes, and a slot is refilled only after the
        compute that read it finished (events).  A helper's result goes back
        to the owner's buffer on the communication stream.  With
        overlap=False every copy runs on the compute stream, in line with
        the computation (the non-overlapped baseline).  Results are bitwise
        those of `forward_items`."""
        items = sorted(self.items_of_worker(w), key=lambda it: it[0])
        if self.n_global > 0:
            raise ValueError("the overlap emulation exchanges whole chunks; global items have none")
        dev = q[w].device
        compute = torch.cuda.current_stream(dev)
        comm = torch.cuda.Stream(dev) if overlap else compute
        # receive slots and the helper's local output, allocated on the
        # compute stream and marked as used by the communication stream
        slots = [{"q": torch.empty_like(q[w]), "k": torch.empty_like(k[w]),
                  "v": torch.empty_like(v[w])} for _ in range(2)]
        helper_out = [self.new_partial(dev) for _ in range(2)]  # double-buffered returns
        back = [None, None]          # return-copy events of each helper buffer
        if overlap:
            for t in [x for sl in slots for x in sl.values()] + [y for h in helper_out for y in h]:
                t.record_stream(comm)
        done = [None, None]          # compute events that last read each slot
        ready = {}                   # step index -> copy-complete event

        def post_copy(i):
            a, c = items[i][2], items[i][3]
            sl = slots[i % 2]
            with torch.cuda.stream(comm):
                if done[i % 2] is not None:
                    comm.wait_event(done[i % 2])
                if a != w:      # helper: the owner's queries come in
                    dfa.dfa_chunk_transfer(sl["q"], q[a], comm)
                elif c != w:    # owner: the key/value chunk comes in
                    dfa.dfa_chunk_transfer(sl["k"], k[c], comm)
                    dfa.dfa_chunk_transfer(sl["v"], v[c], comm)
                ev = torch.cuda.Event()
                ev.record(comm)
                ready[i] = ev

        nh = 0                       # helper items so far
        if items:
            post_copy(0)
        for i, it in enumerate(items):
            if i + 1 < len(items):
                post_copy(i + 1)
            a, c = it[2], it[3]
            sl = slots[i % 2]
            compute.wait_event(ready[i])
            qa = sl["q"] if a != w else q[a]
            kc, vc = (sl["k"], sl["v"]) if (a == w and c != w) else (k[c], v[c])
            if a != w:
                hb = nh % 2
                if back[hb] is not None:
                    compute.wait_event(back[hb])  # its previous result has been sent
                out = helper_out[hb]
            else:
                out = partials[(a, c)]
            d = self.desc(a, c)
            dfa.dfa_attn_fwd_partial(d, qa, kc, vc, *out, None,
                                     self.workspace(d, dfa.DFA_OP_FWD, dev))
            ev = torch.cuda.Event()
            ev.record(compute)
            done[i % 2] = ev
            if a != w:  # send the helper's (O, LSE) back to the owner
                with torch.cuda.stream(comm):
                    comm.wait_event(ev)
                    for dst, src in zip(partials[(a, c)], out):
                        dfa.dfa_chunk_transfer(dst, src, comm)
                    back[hb] = torch.cuda.Event()
                    back[hb].record(comm)
                nh += 1
        if overlap:
            compute.wait_stream(comm)
