"""A Llama-shaped decoder layer (random weights) whose attention is the
chunked causal attention of this library, with three gradient-checkpointing
placements ([DistFlashAttn §3.3]):

  "none"   no checkpointing: autograd keeps every activation;
  "layer"  layer-boundary checkpointing: only the layer input is kept and the
           whole layer, attention forward included, is recomputed in the
           backward, although the attention backward needs only the
           attention output and its LSE;
  "remat"  rematerialisation-aware checkpointing: the layer input and the
           attention output (O and LSE) are kept; the backward recomputes the
           projections and the MLP from them, so the attention forward runs
           once per training step and the numbers are those of "none".

Only the attention runs in this library's kernels; the norms, projections,
rotary embedding and MLP are plain torch operations (library GEMMs).
"""

from __future__ import annotations

import torch
import torch.nn.functional as F

from .autograd import attention_backward, attention_forward, chunked_attention
from .runner import ChunkedCausalAttention

MODES = ("none", "layer", "remat")


def _rms_norm(x, w, eps=1e-6):
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype) * w


def _rotary(x, cos, sin):
    """Rotate the two halves of head_dim by position-dependent angles."""
    half = x.shape[-1] // 2
    xf = x.float()
    x1, x2 = xf[..., :half], xf[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1).to(x.dtype)


class LlamaLayer(torch.nn.Module):
    def __init__(self, att: ChunkedCausalAttention, hidden: int, intermediate: int,
                 device="cuda", seed: int = 0):
        super().__init__()
        self.att = att
        hq, hkv, d = att.heads_q, att.heads_kv, att.head_dim
        dt = torch.bfloat16 if att.dtype == "bf16" else torch.float32
        gen = torch.Generator(device="cpu").manual_seed(seed)

        def w(*shape):
            return torch.nn.Parameter(
                (torch.randn(*shape, generator=gen) * 0.02).to(device=device, dtype=dt))

        self.ln1 = torch.nn.Parameter(torch.ones(hidden, device=device, dtype=dt))
        self.ln2 = torch.nn.Parameter(torch.ones(hidden, device=device, dtype=dt))
        self.wq, self.wk, self.wv = w(hidden, hq * d), w(hidden, hkv * d), w(hidden, hkv * d)
        self.wo = w(hq * d, hidden)
        self.w_gate, self.w_up, self.w_down = w(hidden, intermediate), w(hidden, intermediate), \
            w(intermediate, hidden)
        n = att.workers * att.chunk
        pos = torch.arange(n, dtype=torch.float64)[:, None]
        inv = 10000.0 ** (-torch.arange(0, d // 2, dtype=torch.float64) * 2 / d)[None, :]
        ang = (pos * inv)[None, :, None, :]                      # [1, N, 1, d/2]
        self.register_buffer("cos", ang.cos().float().to(device), persistent=False)
        self.register_buffer("sin", ang.sin().float().to(device), persistent=False)

    # ---- the layer's two halves around the attention ----------------------
    def pre_attn(self, x):
        b, n, _ = x.shape
        att = self.att
        h = _rms_norm(x, self.ln1)
        q = (h @ self.wq).view(b, n, att.heads_q, att.head_dim)
        k = (h @ self.wk).view(b, n, att.heads_kv, att.head_dim)
        v = (h @ self.wv).view(b, n, att.heads_kv, att.head_dim)
        return (_rotary(q, self.cos, self.sin).contiguous(),
                _rotary(k, self.cos, self.sin).contiguous(), v.contiguous())

    def post_attn(self, x, o):
        b, n, _ = x.shape
        y = x + o.reshape(b, n, -1) @ self.wo
        h = _rms_norm(y, self.ln2)
        return y + (F.silu(h @ self.w_gate) * (h @ self.w_up)) @ self.w_down

    def forward(self, x, mode: str = "remat"):
        if mode == "none":
            q, k, v = self.pre_attn(x)
            return self.post_attn(x, chunked_attention(q, k, v, self.att))
        if mode not in MODES:
            raise ValueError(f"mode must be one of {MODES}")
        return _CheckpointedLayer.apply(x, self, mode, *self.parameters())


class _CheckpointedLayer(torch.autograd.Function):
    """Keeps the layer input (and, for "remat", the attention O and LSE);
    recomputes the rest in backward and accumulates the parameter gradients
    into `.grad` directly, like reentrant checkpointing."""

    @staticmethod
    def forward(ctx, x, layer, mode, *params):
        with torch.no_grad():
            q, k, v = layer.pre_attn(x)
            o, lse = attention_forward(layer.att, q, k, v)
            y = layer.post_attn(x, o)
        ctx.layer, ctx.mode = layer, mode
        if mode == "remat":
            ctx.lse = lse
            ctx.save_for_backward(x, o)
        else:
            ctx.save_for_backward(x)
        return y

    @staticmethod
    def backward(ctx, dy):
        layer, att = ctx.layer, ctx.layer.att
        x = ctx.saved_tensors[0]
        with torch.enable_grad():
            x_ = x.detach().requires_grad_(True)
            q, k, v = layer.pre_attn(x_)
            if ctx.mode == "remat":
                o, lse = ctx.saved_tensors[1], ctx.lse
            else:  # layer-boundary: the attention forward runs again
                o, lse = attention_forward(att, q.detach(), k.detach(), v.detach())
            o_ = o.detach().requires_grad_(True)
            y = layer.post_attn(x_, o_)
            torch.autograd.backward(y, dy)
            dq, dk, dv = attention_backward(att, q.detach(), k.detach(), v.detach(), o, lse,
                                            o_.grad)
            torch.autograd.backward((q, k, v), (dq, dk, dv))
        return (x_.grad, None, None) + (None,) * len(tuple(layer.parameters()))


def llama7b_layer(workers: int, chunk: int, device="cuda", seed: int = 0, window: int = 0):
    """Llama-7B's layer shape: hidden 4096, 32 heads of 128, MLP 11008."""
    att = ChunkedCausalAttention(workers, chunk, 1, 32, 32, 128, "bf16", window=window)
    return LlamaLayer(att, 4096, 11008, device, seed)


def layer_flops(att: ChunkedCausalAttention, hidden: int, intermediate: int):
    """Algorithmic FLOP of one forward: (GEMMs, attention over the causal
    pairs at 4d per pair per query head)."""
    n = att.workers * att.chunk
    d, hq, hkv = att.head_dim, att.heads_q, att.heads_kv
    gemm = 2 * n * (hidden * (hq + 2 * hkv) * d + hq * d * hidden + 3 * hidden * intermediate)
    attn = 4 * d * hq * (n * (n + 1) // 2)
    return gemm, attn


__all__ = ["LlamaLayer", "MODES", "llama7b_layer", "layer_flops"]
