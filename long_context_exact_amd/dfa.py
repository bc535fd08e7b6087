"""ctypes binding of libdfa.so, entry point for entry point (see include/dfa.h).

Argument marshalling only: torch tensors become device pointers, the stream
defaults to torch's current stream, shapes / dtypes / devices are checked
against the descriptor before the call (so a mis-shaped tensor can never
reach a kernel), and a non-OK status raises DfaError with the library's
message.  All arithmetic happens in the library's HIP kernels; there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Sequence

import torch

from .build import LIB_PATH

DFA_OK, DFA_ERR_INVALID, DFA_ERR_UNSUPPORTED, DFA_ERR_CAPACITY, DFA_ERR_HIP = range(5)
DFA_F32, DFA_BF16 = 0, 1
DFA_OP_FWD, DFA_OP_BWD = 0, 1
DIAG, FULL, BAND, GLOBAL = 0, 1, 2, 3

_DTYPES = {"f32": DFA_F32, "bf16": DFA_BF16}
_TORCH = {DFA_F32: torch.float32, DFA_BF16: torch.bfloat16}

EXPORTED = (
    "dfa_balanced_schedule", "dfa_window_schedule", "dfa_global_window_schedule",
    "dfa_attn_fwd_partial", "dfa_lse_merge", "dfa_attn_bwd", "dfa_attn_workspace_size",
    "dfa_chunk_transfer", "dfa_attn_fwd_partial_noalloc",
    "dfa_last_error", "dfa_version", "dfa_test_tile_shape", "dfa_test_fwd_tile_visits",
    "dfa_test_bwd_part", "dfa_test_bwd_launches", "dfa_test_work_order",
)


class DfaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[dfa status {status}] {message}")
        self.status = status


class WorkItem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("step", "worker", "q_chunk", "kv_chunk", "kind", "owner")]

    def astuple(self):
        return (self.step, self.worker, self.q_chunk, self.kv_chunk, self.kind, self.owner)


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("len_q", ctypes.c_int64), ("len_kv", ctypes.c_int64),
        ("q_start", ctypes.c_int64), ("kv_start", ctypes.c_int64), ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("window", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


def make_desc(batch, heads_q, heads_kv, head_dim, len_q, len_kv, q_start=0, kv_start=0,
              causal=True, scale=None, dtype="bf16", window=0) -> AttnDesc:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return AttnDesc(int(batch), int(heads_q), int(heads_kv), int(head_dim), int(len_q), int(len_kv),
                    int(q_start), int(kv_start), int(bool(causal)), float(scale),
                    _DTYPES[dtype] if isinstance(dtype, str) else int(dtype), int(window))


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise DfaError(DFA_ERR_HIP, f"{LIB_PATH} is missing: build it with "
                                        "`python -m long_context_exact_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.dfa_balanced_schedule.argtypes = [I32, I32, ctypes.POINTER(WorkItem), I64,
                                            ctypes.POINTER(I64), ctypes.POINTER(I32)]
        L.dfa_window_schedule.argtypes = [I32, I64, I64, ctypes.POINTER(WorkItem), I64,
                                          ctypes.POINTER(I64), ctypes.POINTER(I32)]
        L.dfa_global_window_schedule.argtypes = [I32, I64, I64, I64, ctypes.POINTER(WorkItem), I64,
                                                 ctypes.POINTER(I64), ctypes.POINTER(I32)]
        L.dfa_attn_fwd_partial.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P]
        L.dfa_lse_merge.argtypes = [I32, ctypes.POINTER(P), ctypes.POINTER(P), I32, I32, I64, I32,
                                    I32, P, P, P]
        L.dfa_attn_bwd.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, I32, P, P, P, P]
        L.dfa_test_tile_shape.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(I32),
                                          ctypes.POINTER(I32)]
        L.dfa_test_fwd_tile_visits.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P]
        L.dfa_test_bwd_part.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, I32,
                                        P]
        L.dfa_test_bwd_launches.argtypes = [ctypes.POINTER(AttnDesc), I32, ctypes.POINTER(I32)]
        L.dfa_test_work_order.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(I32),
                                          ctypes.POINTER(I32)]
        L.dfa_attn_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), I32, ctypes.POINTER(I64)]
        L.dfa_chunk_transfer.argtypes = [P, P, I64, P]
        L.dfa_attn_fwd_partial_noalloc.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P]
        for name in ("dfa_balanced_schedule", "dfa_window_schedule", "dfa_global_window_schedule",
                     "dfa_attn_fwd_partial", "dfa_lse_merge", "dfa_attn_workspace_size",
                     "dfa_chunk_transfer", "dfa_attn_fwd_partial_noalloc",
                     "dfa_attn_bwd", "dfa_test_tile_shape", "dfa_test_fwd_tile_visits",
                     "dfa_test_bwd_part", "dfa_test_bwd_launches", "dfa_test_work_order"):
            getattr(L, name).restype = I32
        L.dfa_last_error.argtypes = []
        L.dfa_last_error.restype = ctypes.c_char_p
        L.dfa_version.argtypes = []
        L.dfa_version.restype = I32
        _LIB = L
    return _LIB


def _check(status: int):
    if status != DFA_OK:
        raise DfaError(status, lib().dfa_last_error().decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _torch_stream(stream):
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _ptr(t, name, shape, dtype):
    """Device pointer of a tensor after checking it matches `shape`/`dtype`."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        # the library launches on the current device
        raise ValueError(f"{name} is on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shapes(d: AttnDesc):
    qs = (d.batch, d.len_q, d.heads_q, d.head_dim)
    ks = (d.batch, d.len_kv, d.heads_kv, d.head_dim)
    ls = (d.batch, d.heads_q, d.len_q)
    return qs, ks, ls


def dfa_attn_workspace_size(desc: AttnDesc, op: int) -> int:
    """Bytes of device workspace dfa_attn_fwd_partial (DFA_OP_FWD) or
    dfa_attn_bwd (DFA_OP_BWD) needs for `desc` (host arithmetic only)."""
    n = ctypes.c_int64(0)
    _check(lib().dfa_attn_workspace_size(ctypes.byref(desc), int(op), ctypes.byref(n)))
    return int(n.value)


def _with_workspace(desc: AttnDesc, op: int, workspace, stream):
    """A copy of `desc` naming the caller's workspace (a uint8 device tensor),
    and the tensor to keep alive over the call.  Without one, a workspace of
    the required size is taken from torch's allocator on the call's stream, so
    that torch hands its memory to later work of that stream only."""
    d = AttnDesc.from_buffer_copy(desc)
    if workspace is None:
        need = dfa_attn_workspace_size(desc, op)
        if need == 0:
            d.workspace, d.workspace_bytes = None, 0
            return d, None
        s = _torch_stream(stream)
        with torch.cuda.stream(s):
            workspace = torch.empty(need, dtype=torch.uint8, device=s.device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 torch tensor")
    _ptr(workspace, "workspace", tuple(workspace.shape), torch.uint8)
    d.workspace, d.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return d, workspace


def dfa_version() -> int:
    return int(lib().dfa_version())


def dfa_last_error() -> str:
    return lib().dfa_last_error().decode()


def dfa_balanced_schedule(num_workers: int, balanced: bool = True):
    """(items as tuples (step, worker, q_chunk, kv_chunk, kind, owner), num_steps)."""
    n = ctypes.c_int64(0)
    steps = ctypes.c_int32(0)
    st = lib().dfa_balanced_schedule(int(num_workers), int(bool(balanced)), None, 0,
                                     ctypes.byref(n), ctypes.byref(steps))
    if st not in (DFA_OK, DFA_ERR_CAPACITY):
        _check(st)
    arr = (WorkItem * max(n.value, 1))()
    _check(lib().dfa_balanced_schedule(int(num_workers), int(bool(balanced)), arr, n.value,
                                       ctypes.byref(n), ctypes.byref(steps)))
    return [arr[i].astuple() for i in range(n.value)], int(steps.value)


def dfa_window_schedule(num_workers: int, chunk_len: int, window: int):
    """(items as tuples (step, worker, q_chunk, kv_chunk, kind, owner), num_steps) of the
    sliding-window schedule."""
    n = ctypes.c_int64(0)
    steps = ctypes.c_int32(0)
    st = lib().dfa_window_schedule(int(num_workers), int(chunk_len), int(window), None, 0,
                                   ctypes.byref(n), ctypes.byref(steps))
    if st not in (DFA_OK, DFA_ERR_CAPACITY):
        _check(st)
    arr = (WorkItem * max(n.value, 1))()
    _check(lib().dfa_window_schedule(int(num_workers), int(chunk_len), int(window), arr, n.value,
                                     ctypes.byref(n), ctypes.byref(steps)))
    return [arr[i].astuple() for i in range(n.value)], int(steps.value)


def dfa_global_window_schedule(num_workers: int, chunk_len: int, window: int, n_global: int):
    """(items as tuples, num_steps) of the sliding window plus replicated
    global tokens (global items have kv_chunk -1 and kind GLOBAL)."""
    n = ctypes.c_int64(0)
    steps = ctypes.c_int32(0)
    args = (int(num_workers), int(chunk_len), int(window), int(n_global))
    st = lib().dfa_global_window_schedule(*args, None, 0, ctypes.byref(n), ctypes.byref(steps))
    if st not in (DFA_OK, DFA_ERR_CAPACITY):
        _check(st)
    arr = (WorkItem * max(n.value, 1))()
    _check(lib().dfa_global_window_schedule(*args, arr, n.value, ctypes.byref(n),
                                            ctypes.byref(steps)))
    return [arr[i].astuple() for i in range(n.value)], int(steps.value)


def dfa_attn_fwd_partial(desc: AttnDesc, q, k, v, o_part, lse, stream=None, workspace=None):
    """workspace: a uint8 device tensor of at least
    dfa_attn_workspace_size(desc, DFA_OP_FWD) bytes (taken from torch's
    allocator for this call when None)."""
    qs, ks, ls = _shapes(desc)
    dt = _TORCH.get(desc.dtype, torch.bfloat16)
    args = (_ptr(q, "q", qs, dt), _ptr(k, "k", ks, dt), _ptr(v, "v", ks, dt),
            _ptr(o_part, "o_part", qs, torch.float32), _ptr(lse, "lse", ls, torch.float32))
    d, _keep = _with_workspace(desc, DFA_OP_FWD, workspace, stream)
    _check(lib().dfa_attn_fwd_partial(ctypes.byref(d), *args, _stream(stream)))


def dfa_attn_fwd_partial_noalloc(desc: AttnDesc, q, k, v, o_part, lse, stream=None):
    """dfa_attn_fwd_partial with its scratch in the library's fixed per-device
    array: allocates nothing (for code that cannot allocate)."""
    qs, ks, ls = _shapes(desc)
    dt = _TORCH.get(desc.dtype, torch.bfloat16)
    args = (_ptr(q, "q", qs, dt), _ptr(k, "k", ks, dt), _ptr(v, "v", ks, dt),
            _ptr(o_part, "o_part", qs, torch.float32), _ptr(lse, "lse", ls, torch.float32))
    _check(lib().dfa_attn_fwd_partial_noalloc(ctypes.byref(desc), *args, _stream(stream)))


def dfa_lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], batch: int,
                  heads: int, len_q: int, head_dim: int, out_dtype, o_out, lse_out, stream=None):
    n = len(o_parts)
    if n != len(lse_parts):
        raise ValueError("o_parts and lse_parts differ in length")
    od = _DTYPES[out_dtype] if isinstance(out_dtype, str) else int(out_dtype)
    os_ = (batch, len_q, heads, head_dim)
    ls = (batch, heads, len_q)
    op = (ctypes.c_void_p * max(n, 1))(*[_ptr(t, f"o_parts[{i}]", os_, torch.float32)
                                         for i, t in enumerate(o_parts)])
    lp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t, f"lse_parts[{i}]", ls, torch.float32)
                                         for i, t in enumerate(lse_parts)])
    _check(lib().dfa_lse_merge(n, op, lp, int(batch), int(heads), int(len_q), int(head_dim), od,
                               _ptr(o_out, "o_out", os_, _TORCH.get(od, torch.float32)),
                               _ptr(lse_out, "lse_out", ls, torch.float32), _stream(stream)))


def dfa_attn_bwd(desc: AttnDesc, q, k, v, o, lse, d_o, delta, compute_delta: bool, dq, dk, dv,
                 stream=None, workspace=None):
    """workspace: a uint8 device tensor of at least
    dfa_attn_workspace_size(desc, DFA_OP_BWD) bytes (taken from torch's
    allocator for this call when None and needed)."""
    qs, ks, ls = _shapes(desc)
    dt = _TORCH.get(desc.dtype, torch.bfloat16)
    f32 = torch.float32
    args = (_ptr(q, "q", qs, dt), _ptr(k, "k", ks, dt), _ptr(v, "v", ks, dt),
            _ptr(o, "o", qs, dt), _ptr(lse, "lse", ls, f32), _ptr(d_o, "d_o", qs, dt),
            _ptr(delta, "delta", ls, f32), int(bool(compute_delta)),
            _ptr(dq, "dq", qs, f32), _ptr(dk, "dk", ks, f32), _ptr(dv, "dv", ks, f32))
    d, _keep = _with_workspace(desc, DFA_OP_BWD, workspace, stream)
    _check(lib().dfa_attn_bwd(ctypes.byref(d), *args, _stream(stream)))


def dfa_chunk_transfer(dst, src, stream=None):
    """dst <- src (same shape and dtype, contiguous, on the current device)
    on a DMA engine, enqueued on `stream`: the emulated exchange of a chunk."""
    if not isinstance(src, torch.Tensor):
        raise TypeError("src must be a torch.Tensor")
    s_ptr = _ptr(src, "src", tuple(src.shape), src.dtype)
    d_ptr = _ptr(dst, "dst", tuple(src.shape), src.dtype)
    _check(lib().dfa_chunk_transfer(d_ptr, s_ptr, src.numel() * src.element_size(),
                                    _stream(stream)))


def dfa_test_tile_shape(desc: AttnDesc):
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().dfa_test_tile_shape(ctypes.byref(desc), ctypes.byref(bm), ctypes.byref(bn)))
    return int(bm.value), int(bn.value)


def dfa_test_fwd_tile_visits(desc: AttnDesc, q, k, v, o_part, lse, visits, stream=None,
                             workspace=None):
    qs, ks, ls = _shapes(desc)
    bm, bn = dfa_test_tile_shape(desc)
    vshape = (-(-desc.len_q // bm), -(-desc.len_kv // bn))
    dt = _TORCH.get(desc.dtype, torch.bfloat16)
    args = (_ptr(q, "q", qs, dt), _ptr(k, "k", ks, dt), _ptr(v, "v", ks, dt),
            _ptr(o_part, "o_part", qs, torch.float32), _ptr(lse, "lse", ls, torch.float32),
            _ptr(visits, "visits", vshape, torch.uint8))
    d, _keep = _with_workspace(desc, DFA_OP_FWD, workspace, stream)
    _check(lib().dfa_test_fwd_tile_visits(ctypes.byref(d), *args, _stream(stream)))


def dfa_test_bwd_launches(desc: AttnDesc, part: int) -> int:
    """Kernel launches dfa_test_bwd_part makes for `part` (host only)."""
    n = ctypes.c_int32(-1)
    _check(lib().dfa_test_bwd_launches(ctypes.byref(desc), int(part), ctypes.byref(n)))
    return n.value


def dfa_test_work_order(desc: AttnDesc):
    """(rows first to last, dK/dV key blocks last to first) for the pair (host only)."""
    r, k = ctypes.c_int32(-1), ctypes.c_int32(-1)
    _check(lib().dfa_test_work_order(ctypes.byref(desc), ctypes.byref(r), ctypes.byref(k)))
    return bool(r.value), bool(k.value)


def dfa_test_bwd_part(desc: AttnDesc, q, k, v, lse, d_o, delta, dq, dk, dv, part: int,
                      stream=None, workspace=None):
    """One backward kernel alone (1: dK/dV, 2: dQ), delta already computed."""
    qs, ks, ls = _shapes(desc)
    dt = _TORCH.get(desc.dtype, torch.bfloat16)
    f32 = torch.float32
    args = (_ptr(q, "q", qs, dt), _ptr(k, "k", ks, dt), _ptr(v, "v", ks, dt),
            _ptr(lse, "lse", ls, f32), _ptr(d_o, "d_o", qs, dt), _ptr(delta, "delta", ls, f32),
            _ptr(dq, "dq", qs, f32) if part == 2 else None,
            _ptr(dk, "dk", ks, f32) if part == 1 else None,
            _ptr(dv, "dv", ks, f32) if part == 1 else None)
    d, _keep = _with_workspace(desc, DFA_OP_BWD, workspace, stream)
    _check(lib().dfa_test_bwd_part(ctypes.byref(d), *args, int(part), _stream(stream)))
