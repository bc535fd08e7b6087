"""The seeded input generator: reproducible per (seed, tensor, chunk) and its
bfloat16 rounding equal to torch's round-to-nearest-even conversion."""

import numpy as np
import torch

from long_context_exact_amd.synth import WORKLOADS, bf16_bits, bf16_round, chunk_tensor


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], np.float32)])
    # exact ties in both directions
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(x), ref)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(bf16_round(x)), bits)


def test_chunks_are_reproducible_and_distinct():
    a = chunk_tensor(5, 0, 3, (1, 64, 2, 8), "bf16")
    b = chunk_tensor(5, 0, 3, (1, 64, 2, 8), "bf16")
    c = chunk_tensor(5, 1, 3, (1, 64, 2, 8), "bf16")
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(bf16_round(a), a)


def test_workload_shapes():
    w = WORKLOADS["gqa64x8_512k_w15"]
    assert w.total_len == 524288 and w.q_shape() == (1, 32768, 64, 128)
    assert w.kv_shape() == (1, 32768, 8, 128)
    assert WORKLOADS["tiny_f32"].total_len == 512
