"""Helpers shared by the GPU parity tests: seeded inputs, running the whole
chunked path through the C ABI, and the tolerance checks.

Tolerances (float64 oracle as the truth):
  fp32 inputs: max |err| <= 1e-5 on O, LSE, dQ, dK, dV.
  bf16 inputs, fp32 accumulation: O max |err| <= 1e-2 (an O delivered in
  bf16 is allowed, on top, the rounding of the exact value to bf16: half a
  bf16 spacing, 2**(e - 8) for |x| in [2**e, 2**(e + 1))); LSE relative <= 1e-3;
  dQ, dK, dV relative Frobenius <= 2e-2; plus an internal guard of
  relative Frobenius <= 2e-2 on O (O shrinks like 1/sqrt(prefix) at long
  contexts, where 1e-2 absolute would be loose).
"""

from __future__ import annotations

import zlib

import numpy as np
import torch

from long_context_exact_amd.runner import ChunkedCausalAttention
from long_context_exact_amd.synth import bf16_round

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
DEV = "cuda"


def rand(rng, shape, dtype, scale=1.0):
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def case_seed(case) -> int:
    """A seed that is the same in every process (Python's hash of strings is not)."""
    return zlib.crc32(repr(case).encode())


def bf16_half_spacing(x: np.ndarray) -> np.ndarray:
    """Half the gap between neighbouring bf16 values at |x| (0 at x = 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(TD[dtype])


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_fro(a, b):
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def check_o(o, ref, dtype, what="O", stored_bf16=False):
    """`stored_bf16`: o is the output as delivered in bf16, so each element
    may also differ from the exact value by the rounding to bf16."""
    err = float(np.max(np.abs(o - ref))) if o.size else 0.0
    if dtype == "f32":
        assert err <= 1e-5, f"{what}: max abs err {err}"
    else:
        if stored_bf16 and o.size:
            excess = float(np.max(np.abs(o - ref) - bf16_half_spacing(ref)))
            assert excess <= 1e-2, f"{what}: max abs err {err} ({excess} beyond bf16 rounding)"
        else:
            assert err <= 1e-2, f"{what}: max abs err {err}"
        assert rel_fro(o, ref) <= 2e-2, f"{what}: rel fro {rel_fro(o, ref)}"


def check_lse(lse, ref, dtype, what="LSE"):
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite values"
    if not fin.any():
        return
    d = np.abs(lse[fin] - ref[fin])
    if dtype == "f32":
        assert float(d.max()) <= 1e-5, f"{what}: max abs err {float(d.max())}"
    else:
        strict = d / np.maximum(np.abs(ref[fin]), 1e-300)
        # relative error of a value near zero is ill-conditioned (the
        # absolute error of an LSE scales with its summands, not with the
        # LSE): where |LSE| < 1 the same 1e-3 bound is applied absolutely
        rel = np.where(np.abs(ref[fin]) < 1.0, d, strict)
        if float(strict.max()) > 1e-3:  # visible in the test output
            print(f"{what}: strict relative error {float(strict.max()):.3e} at |LSE| = "
                  f"{float(np.abs(ref[fin])[np.argmax(strict)]):.3e}; held to 1e-3 absolute "
                  f"there (max {float(rel.max()):.3e})", flush=True)
        assert float(rel.max()) <= 1e-3, f"{what}: rel err {float(rel.max())}"


def check_grad(g, ref, dtype, what):
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    if dtype == "f32":
        err = float(np.max(np.abs(g - ref)))
        assert err <= 1e-5, f"{what}: max abs err {err}"
    else:
        r = rel_fro(g, ref)
        assert r <= 2e-2, f"{what}: rel fro {r}"


def run_sequence(att: ChunkedCausalAttention, q, k, v, d_o=None):
    """All pairs of the schedule, every owner's merge and (if d_o) the whole
    backward.  q, k, v, d_o: lists of per-chunk numpy arrays (already
    representable in the dtype).  Returns numpy float64 results keyed like
    the runner's buffers."""
    P, dt = att.workers, att.dtype
    qd = {a: to_dev(q[a], dt) for a in range(P)}
    kd = {a: to_dev(k[a], dt) for a in range(P)}
    vd = {a: to_dev(v[a], dt) for a in range(P)}
    partials = {(it[2], it[3]): att.new_partial() for it in att.items}
    att.forward_items(att.items, qd, kd, vd, partials)
    o = {a: torch.empty(att.q_shape(), dtype=TD[dt], device=DEV) for a in range(P)}
    lse = {a: torch.empty(att.lse_shape(), dtype=torch.float32, device=DEV) for a in range(P)}
    for a in range(P):
        att.merge_owner(a, partials, o[a], lse[a])
    out = {"partials": {key: (to_np(x), to_np(y)) for key, (x, y) in partials.items()},
           "o": [to_np(o[a]) for a in range(P)], "lse": [to_np(lse[a]) for a in range(P)],
           "o_dev": o, "lse_dev": lse}
    if d_o is not None:
        dod = {a: to_dev(d_o[a], dt) for a in range(P)}
        dq = {a: torch.zeros(att.q_shape(), dtype=torch.float32, device=DEV) for a in range(P)}
        dk = {a: torch.zeros(att.kv_shape(), dtype=torch.float32, device=DEV) for a in range(P)}
        dv = {a: torch.zeros(att.kv_shape(), dtype=torch.float32, device=DEV) for a in range(P)}
        delta = {a: torch.empty(att.lse_shape(), dtype=torch.float32, device=DEV) for a in range(P)}
        att.backward_items(att.items, qd, kd, vd, o, lse, dod, delta, dq, dk, dv)
        out.update(dq=[to_np(dq[a]) for a in range(P)], dk=[to_np(dk[a]) for a in range(P)],
                   dv=[to_np(dv[a]) for a in range(P)], delta=[to_np(delta[a]) for a in range(P)])
    torch.cuda.synchronize()
    return out
