"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module holds no attention arithmetic: it draws i.i.d. N(0, 1) tensors
chunk by chunk from a counter-keyed numpy generator and, for bfloat16
workloads, rounds them to the nearest bfloat16 (ties to even) so that the
GPU receives exactly the bits whose float64 upcast the oracle receives.

The paper trains Llama-7B-shaped models (32 heads of 128; abstract, §4.1)
on sequences of 32K-512K tokens split over P workers (§3.1, §4.5); no
dataset is needed for the attention hot path, so standard-normal Q, K, V
and dO stand in for real activations (scores then have unit variance with
scale 1/sqrt(d)).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; the result
    is float32 holding exactly representable bfloat16 values.  Inputs here
    are finite normal draws, so NaN handling is not needed (and not done)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def chunk_tensor(seed: int, tensor_id: int, chunk: int, shape, dtype: str) -> np.ndarray:
    """One chunk of one input tensor, float32, shape e.g. (B, C, H, d).

    The generator is keyed by (seed, tensor_id, chunk) so any chunk can be
    drawn on its own (a worker's share needs only its own query chunk and the
    key/value chunks it reads)."""
    rng = np.random.default_rng([int(seed), int(tensor_id), int(chunk)])
    x = rng.standard_normal(tuple(int(s) for s in shape), dtype=np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


@dataclass(frozen=True)
class Workload:
    """One attention workload: B x (P chunks of C tokens) x heads x head_dim."""
    name: str
    chunk: int          # C, tokens per worker chunk
    workers: int        # P
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    seed: int
    backward: bool      # fwd + bwd (True) or fwd only
    share_of: int       # -1: every chunk pair; w: worker w's share only
    batch: int = 1
    window: int = 0     # 0: full causal attention; > 0: local sliding window (tokens)
    n_global: int = 0   # > 0 (with a window): the first n_global tokens are global

    @property
    def total_len(self) -> int:
        return self.chunk * self.workers

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def q_shape(self, length=None):
        return (self.batch, self.chunk if length is None else length, self.heads_q, self.head_dim)

    def kv_shape(self, length=None):
        return (self.batch, self.chunk if length is None else length, self.heads_kv, self.head_dim)

    def chunk_input(self, tensor_id: int, chunk: int) -> np.ndarray:
        shape = self.kv_shape() if tensor_id in (TENSOR_K, TENSOR_V) else self.q_shape()
        return chunk_tensor(self.seed, tensor_id, chunk, shape, self.dtype)


# The workloads: a tiny fp32 case, three Llama-7B-shaped (32 x 128) bf16
# cases, a grouped-query (64 query heads over 8 key/value heads) worker share
# at a 32768-token chunk, and that share under a local sliding window.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 128, 4, 2, 2, 64, "f32", 1001, True, -1),
    "llama7b_32k_fwd": Workload("llama7b_32k_fwd", 4096, 8, 32, 32, 128, "bf16", 1002, False, -1),
    "llama7b_64k": Workload("llama7b_64k", 8192, 8, 32, 32, 128, "bf16", 1003, True, -1),
    "llama7b_256k_w15": Workload("llama7b_256k_w15", 16384, 16, 32, 32, 128, "bf16", 1004, True, 15),
    "gqa64x8_512k_w15": Workload("gqa64x8_512k_w15", 32768, 16, 64, 8, 128, "bf16", 1005, True, 15),
    # the same worker share under a local sliding window of 4096 tokens
    "gqa64x8_512k_win4k_w15": Workload("gqa64x8_512k_win4k_w15", 32768, 16, 64, 8, 128, "bf16",
                                       1006, True, 15, window=4096),
    # and with the first 1024 tokens global (replicated on every worker)
    "gqa64x8_512k_win4k_g1k_w15": Workload("gqa64x8_512k_win4k_g1k_w15", 32768, 16, 64, 8, 128,
                                           "bf16", 1007, True, 15, window=4096, n_global=1024),
}
