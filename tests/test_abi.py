"""CPU checks of the C ABI: the library loads and exports every function the
header declares, the schedule is bit-exact against the oracle's, and every
argument check fails cleanly (before any GPU work) with the documented
status."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle
from long_context_exact_amd import dfa as D

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dfa.h")
FAKE = ctypes.c_void_p(1 << 20)      # never dereferenced: each call below fails validation


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(dfa_lib):
    names = _declared()
    assert set(names) == set(D.EXPORTED)
    L = dfa_lib.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", D.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_version(dfa_lib):
    assert dfa_lib.dfa_version() == 10100


@pytest.mark.parametrize("p", list(range(1, 65)) + [127, 128, 1000])
@pytest.mark.parametrize("balanced", [True, False])
def test_schedule_bit_exact_vs_oracle(dfa_lib, p, balanced):
    items, steps = dfa_lib.dfa_balanced_schedule(p, balanced)
    ref, ref_steps = (oracle.balanced_schedule if balanced else oracle.unbalanced_schedule)(p)
    assert steps == ref_steps
    assert items == [tuple(x) for x in ref]


def test_schedule_argument_errors(dfa_lib):
    L = dfa_lib.lib()
    n, s = ctypes.c_int64(-1), ctypes.c_int32(-1)
    assert L.dfa_balanced_schedule(0, 1, None, 0, ctypes.byref(n), ctypes.byref(s)) == D.DFA_ERR_INVALID
    assert "num_workers" in dfa_lib.dfa_last_error()
    assert L.dfa_balanced_schedule(4, 2, None, 0, ctypes.byref(n), ctypes.byref(s)) == D.DFA_ERR_INVALID
    assert L.dfa_balanced_schedule(4, 1, None, 0, None, ctypes.byref(s)) == D.DFA_ERR_INVALID
    arr = (D.WorkItem * 3)()
    assert L.dfa_balanced_schedule(4, 1, arr, 3, ctypes.byref(n), ctypes.byref(s)) == D.DFA_ERR_CAPACITY
    assert n.value == 10 and s.value == 3
    assert L.dfa_balanced_schedule(4, 1, None, 0, ctypes.byref(n), ctypes.byref(s)) == D.DFA_ERR_CAPACITY
    assert n.value == 10


@pytest.mark.parametrize("p", [1, 2, 3, 8, 16, 33])
@pytest.mark.parametrize("c", [1, 7, 128, 32768])
@pytest.mark.parametrize("win_of_c", [0.001, 0.5, 1.0, 1.5, 2.0, 5.25])
def test_window_schedule_bit_exact_vs_oracle(dfa_lib, p, c, win_of_c):
    win = max(1, int(win_of_c * c))
    for w_ in {win, win + 1, max(1, win - 1)}:
        items, steps = dfa_lib.dfa_window_schedule(p, c, w_)
        ref, ref_steps = oracle.window_schedule(p, c, w_)
        assert steps == ref_steps
        assert items == [tuple(x) for x in ref]


def test_window_schedule_argument_errors(dfa_lib):
    L = dfa_lib.lib()
    n, s = ctypes.c_int64(-1), ctypes.c_int32(-1)
    for args in ((0, 4, 4), (4, 0, 4), (4, 4, 0), (70000, 4, 4)):
        assert L.dfa_window_schedule(*args, None, 0, ctypes.byref(n), ctypes.byref(s)) == \
            D.DFA_ERR_INVALID
        assert dfa_lib.dfa_last_error().startswith("dfa_window_schedule")
    arr = (D.WorkItem * 3)()
    assert L.dfa_window_schedule(8, 4, 4, arr, 3, ctypes.byref(n), ctypes.byref(s)) == \
        D.DFA_ERR_CAPACITY
    assert n.value == 15 and s.value == 2


@pytest.mark.parametrize("p", [1, 2, 5, 16])
@pytest.mark.parametrize("c", [1, 7, 128, 32768])
@pytest.mark.parametrize("win_of_c", [0.001, 0.5, 1.0, 2.5])
@pytest.mark.parametrize("g_of_c", [0.0, 0.03, 0.5, 1.0])
def test_global_window_schedule_bit_exact_vs_oracle(dfa_lib, p, c, win_of_c, g_of_c):
    win = max(1, int(win_of_c * c))
    g = min(c, max(1, int(g_of_c * c)))
    items, steps = dfa_lib.dfa_global_window_schedule(p, c, win, g)
    ref, ref_steps = oracle.global_window_schedule(p, c, win, g)
    assert steps == ref_steps
    assert items == [tuple(x) for x in ref]


def test_global_window_schedule_argument_errors(dfa_lib):
    L = dfa_lib.lib()
    n, s = ctypes.c_int64(-1), ctypes.c_int32(-1)
    for args in ((0, 4, 4, 1), (4, 0, 4, 1), (4, 4, 0, 1), (4, 4, 4, 0), (4, 4, 4, 5),
                 (70000, 4, 4, 1)):
        assert L.dfa_global_window_schedule(*args, None, 0, ctypes.byref(n), ctypes.byref(s)) == \
            D.DFA_ERR_INVALID
        assert dfa_lib.dfa_last_error().startswith("dfa_global_window_schedule")
    arr = (D.WorkItem * 3)()
    # 8 global items + the window schedule's 15
    assert L.dfa_global_window_schedule(8, 4, 4, 2, arr, 3, ctypes.byref(n), ctypes.byref(s)) == \
        D.DFA_ERR_CAPACITY
    assert n.value == 23 and s.value == 2


def _fwd(L, d, q=FAKE, o=FAKE, lse=FAKE):
    return L.dfa_attn_fwd_partial(ctypes.byref(d) if d is not None else None, q, FAKE, FAKE, o,
                                  lse, None)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, D.DFA_ERR_UNSUPPORTED),
    ("head_dim", 256, D.DFA_ERR_UNSUPPORTED),
    ("heads_q", 3, D.DFA_ERR_INVALID),        # not a multiple of heads_kv = 2
    ("heads_kv", 0, D.DFA_ERR_INVALID),
    ("len_q", -1, D.DFA_ERR_INVALID),
    ("kv_start", -5, D.DFA_ERR_INVALID),
    ("causal", 2, D.DFA_ERR_INVALID),
    ("scale", -0.5, D.DFA_ERR_INVALID),
    ("scale", float("inf"), D.DFA_ERR_INVALID),
    ("dtype", 7, D.DFA_ERR_INVALID),
    ("batch", -1, D.DFA_ERR_INVALID),
    ("window", -1, D.DFA_ERR_INVALID),
    ("heads_q", 16384, D.DFA_ERR_UNSUPPORTED),  # 16384 * 128 = 2^21: past 32-bit tile offsets
])
def test_fwd_descriptor_errors(dfa_lib, field, value, status):
    L = dfa_lib.lib()
    d = D.make_desc(1, 4, 2, 128, 256, 256)
    setattr(d, field, value)
    assert _fwd(L, d) == status
    assert dfa_lib.dfa_last_error().startswith("dfa_attn_fwd_partial")


def test_window_needs_causal(dfa_lib):
    L = dfa_lib.lib()
    d = D.make_desc(1, 4, 2, 128, 256, 256, causal=False, window=64)
    assert _fwd(L, d) == D.DFA_ERR_INVALID
    assert "window" in dfa_lib.dfa_last_error()


def test_fwd_pointer_errors(dfa_lib):
    L = dfa_lib.lib()
    d = D.make_desc(1, 4, 2, 128, 256, 256)
    assert _fwd(L, None) == D.DFA_ERR_INVALID
    assert _fwd(L, d, q=None) == D.DFA_ERR_INVALID
    assert _fwd(L, d, lse=None) == D.DFA_ERR_INVALID
    assert _fwd(L, d, o=ctypes.c_void_p((1 << 20) + 4)) == D.DFA_ERR_INVALID   # misaligned
    assert "aligned" in dfa_lib.dfa_last_error()


def test_empty_problems_enqueue_nothing(dfa_lib):
    """len_q == 0 and batch == 0 return OK without touching the runtime, so
    they succeed even with no GPU present."""
    L = dfa_lib.lib()
    assert _fwd(L, D.make_desc(1, 2, 2, 64, 0, 128), q=None, o=None, lse=None) == D.DFA_OK
    assert _fwd(L, D.make_desc(0, 2, 2, 64, 16, 128), q=None, o=None, lse=None) == D.DFA_OK


def test_merge_errors(dfa_lib):
    L = dfa_lib.lib()
    P = ctypes.c_void_p
    two = (P * 2)(FAKE, P((1 << 20) + 4096))
    lses = (P * 2)(FAKE, P((1 << 20) + 8192))

    def merge(n=2, o=two, l=lses, heads=2, hd=64, od=D.DFA_F32, out=P((1 << 21)), lout=P(1 << 22)):
        return L.dfa_lse_merge(n, o, l, 1, heads, 16, hd, od, out, lout, None)

    assert merge(n=0) == D.DFA_ERR_INVALID
    assert merge(n=65) == D.DFA_ERR_INVALID
    assert merge(o=None) == D.DFA_ERR_INVALID
    assert merge(hd=80) == D.DFA_ERR_UNSUPPORTED
    assert merge(od=5) == D.DFA_ERR_INVALID
    assert merge(heads=0) == D.DFA_ERR_INVALID
    assert merge(out=two[1]) == D.DFA_ERR_INVALID                 # aliases o_parts[1]
    assert merge(out=two[0], od=D.DFA_BF16) == D.DFA_ERR_INVALID  # bf16 over fp32 input
    assert merge(lout=lses[1]) == D.DFA_ERR_INVALID
    assert "alias" in dfa_lib.dfa_last_error()


def test_bwd_errors(dfa_lib):
    L = dfa_lib.lib()
    d = D.make_desc(1, 2, 2, 64, 64, 64)

    def bwd(desc=d, cd=1, o=FAKE, dq=FAKE):
        return L.dfa_attn_bwd(ctypes.byref(desc), FAKE, FAKE, FAKE, o, FAKE, FAKE, FAKE, cd, dq,
                              FAKE, FAKE, None)

    assert bwd(cd=3) == D.DFA_ERR_INVALID
    assert bwd(o=None) == D.DFA_ERR_INVALID        # compute_delta needs o
    assert bwd(dq=None) == D.DFA_ERR_INVALID
    d2 = D.make_desc(1, 2, 2, 32, 64, 64)
    assert bwd(desc=d2) == D.DFA_ERR_UNSUPPORTED


def test_tile_shape_and_visit_guards(dfa_lib):
    d = D.make_desc(1, 64, 8, 128, 32768, 32768)
    bm, bn = dfa_lib.dfa_test_tile_shape(d)
    assert bm >= 32 and bm % 32 == 0 and bn % 32 == 0
    L = dfa_lib.lib()
    f = D.make_desc(1, 2, 2, 64, 128, 128, dtype="f32")
    assert L.dfa_test_fwd_tile_visits(ctypes.byref(f), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None) == D.DFA_ERR_UNSUPPORTED
    assert L.dfa_test_fwd_tile_visits(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                      None) == D.DFA_ERR_INVALID


def test_runtime_without_device_reports_hip_error(dfa_lib):
    """With a valid call and no GPU, the launch fails with DFA_ERR_HIP (no
    crash, no exception across the ABI).  Skipped where a GPU exists: the
    pointers here are fake."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = dfa_lib.lib()
    d = D.make_desc(1, 2, 2, 64, 128, 128)
    d.workspace, d.workspace_bytes = 1 << 24, 1 << 20
    assert _fwd(L, d) == D.DFA_ERR_HIP
    assert dfa_lib.dfa_last_error()


def test_binding_rejects_mismatched_tensors(dfa_lib):
    import torch
    d = D.make_desc(1, 2, 2, 64, 16, 16)
    cpu = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        dfa_lib.dfa_attn_fwd_partial(d, cpu, cpu, cpu, None, None)


def _ws_size(dfa_lib, d, op):
    n = ctypes.c_int64(-1)
    st = dfa_lib.lib().dfa_attn_workspace_size(ctypes.byref(d), op, ctypes.byref(n))
    return st, n.value


def test_workspace_size_forward(dfa_lib):
    """The forward's workspace is the transposed V: 2 bytes per element of
    [B][Hkv][d][keys rounded up to 128]; nothing for fp32 or empty pairs."""
    for b, hq, hkv, dh, lq, lk in ((1, 64, 8, 128, 32768, 32768), (2, 4, 2, 64, 100, 130),
                                   (3, 6, 3, 128, 1, 1)):
        d = D.make_desc(b, hq, hkv, dh, lq, lk)
        st, n = _ws_size(dfa_lib, d, D.DFA_OP_FWD)
        assert st == D.DFA_OK and n == 2 * b * hkv * dh * (-(-lk // 128) * 128)
        assert dfa_lib.dfa_attn_workspace_size(d, D.DFA_OP_FWD) == n
    assert dfa_lib.dfa_attn_workspace_size(D.make_desc(1, 2, 2, 64, 128, 128, dtype="f32"),
                                           D.DFA_OP_FWD) == 0
    assert dfa_lib.dfa_attn_workspace_size(D.make_desc(1, 2, 2, 64, 0, 128), D.DFA_OP_FWD) == 0
    assert dfa_lib.dfa_attn_workspace_size(D.make_desc(1, 2, 2, 64, 16, 0), D.DFA_OP_FWD) == 0
    assert dfa_lib.dfa_attn_workspace_size(D.make_desc(1, 64, 8, 128, 32768, 32768),
                                           D.DFA_OP_FWD) == 64 << 20   # the 32K-chunk GQA pair


def test_workspace_size_backward():
    """The backward needs scratch only where dK/dV splits a key block's rows:
    not on whole-chunk pairs, but on a short key range against a long query
    chunk (the 1024 global keys against a 32768-row chunk: 8 slices of fp32
    dK and dV) and on a window band."""
    per = 2 * 1024 * 8 * 128 * 4          # one slice: fp32 dK and dV of 1024 keys x 8 heads
    for lq, lk, qs, ks, win, want in ((32768, 32768, 15 * 32768, 14 * 32768, 0, 0),
                                      (32768, 32768, 15 * 32768, 15 * 32768, 0, 0),
                                      (32768, 1024, 15 * 32768, 0, 0, 8 * per)):
        d = D.make_desc(1, 64, 8, 128, lq, lk, qs, ks, window=win)
        assert D.dfa_attn_workspace_size(d, D.DFA_OP_BWD) == want, (lq, lk, win)
    band = D.make_desc(1, 64, 8, 128, 32768, 32768, 15 * 32768, 14 * 32768, window=4096)
    n = D.dfa_attn_workspace_size(band, D.DFA_OP_BWD)
    assert n > 0 and n % (2 * 32768 * 8 * 128 * 4) == 0 and n <= 4 << 30
    assert D.dfa_attn_workspace_size(D.make_desc(1, 2, 2, 64, 4096, 64, dtype="f32"),
                                     D.DFA_OP_BWD) == 0


def test_bwd_launch_counts(dfa_lib):
    """dK/dV runs a diagonal pair of whole 256-key blocks as two row-band
    launches (with a window of >= 512 rows, a multiple of 32, shorter than
    the chunk, the first pairs each block's own rows with its window-edge
    rows) and everything else as one launch; dQ is always one launch; a pair
    without rows or keys launches nothing."""
    C = 32768
    n = D.dfa_test_bwd_launches
    full = D.make_desc(1, 64, 8, 128, C, C, 15 * C, 14 * C)
    diag = D.make_desc(1, 64, 8, 128, C, C, 15 * C, 15 * C)
    assert (n(full, 1), n(full, 2), n(diag, 1), n(diag, 2)) == (1, 1, 2, 1)
    for win, want in ((4096, 2), (512, 2), (C, 2), (1 << 40, 2), (500, 1), (256, 1), (480, 1)):
        d = D.make_desc(1, 64, 8, 128, C, C, 15 * C, 15 * C, window=win)
        assert n(d, 1) == want, win
    # a band pair of a window (not diagonal), a ragged diagonal, head_dim 64
    assert n(D.make_desc(1, 64, 8, 128, C, C, 15 * C, 14 * C, window=4096), 1) == 1
    assert n(D.make_desc(1, 8, 2, 128, 1000, 1000), 1) == 1
    d64 = D.make_desc(1, 32, 8, 64, 16384, 16384)
    assert D.dfa_attn_workspace_size(d64, D.DFA_OP_BWD) == 0 and n(d64, 1) == 2
    # a diagonal whose rows the dK/dV kernel splits over workgroups does not band
    split = D.make_desc(1, 8, 1, 128, 512, 512)
    assert D.dfa_attn_workspace_size(split, D.DFA_OP_BWD) > 0 and n(split, 1) == 1
    assert n(D.make_desc(1, 8, 2, 64, 1024, 1024, dtype="f32"), 1) == 1
    for lq, lk in ((0, 256), (256, 0)):
        e = D.make_desc(1, 4, 2, 128, lq, lk)
        assert (n(e, 1), n(e, 2)) == (0, 0)
    L = dfa_lib.lib()
    c = ctypes.c_int32(0)
    assert L.dfa_test_bwd_launches(ctypes.byref(diag), 3, ctypes.byref(c)) == D.DFA_ERR_INVALID
    assert L.dfa_test_bwd_launches(ctypes.byref(diag), 1, None) == D.DFA_ERR_INVALID
    assert L.dfa_test_bwd_launches(None, 1, ctypes.byref(c)) == D.DFA_ERR_INVALID


def test_workspace_size_errors(dfa_lib):
    L = dfa_lib.lib()
    d = D.make_desc(1, 4, 2, 128, 256, 256)
    n = ctypes.c_int64(0)
    assert L.dfa_attn_workspace_size(ctypes.byref(d), 2, ctypes.byref(n)) == D.DFA_ERR_INVALID
    assert L.dfa_attn_workspace_size(ctypes.byref(d), 0, None) == D.DFA_ERR_INVALID
    assert L.dfa_attn_workspace_size(None, 0, ctypes.byref(n)) == D.DFA_ERR_INVALID
    d.head_dim = 96
    assert L.dfa_attn_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == D.DFA_ERR_UNSUPPORTED


def test_undersized_workspace_is_a_capacity_error(dfa_lib):
    """A workspace smaller than the query's answer (or none) fails with
    DFA_ERR_CAPACITY naming the required size, before anything is enqueued
    (the pointers are fake; no GPU is touched)."""
    L = dfa_lib.lib()
    d = D.make_desc(1, 4, 2, 128, 256, 300)
    need = dfa_lib.dfa_attn_workspace_size(d, D.DFA_OP_FWD)
    assert need == 2 * 2 * 128 * 384
    assert _fwd(L, d) == D.DFA_ERR_CAPACITY                       # no workspace
    assert f"{need} bytes required" in dfa_lib.dfa_last_error()
    d.workspace, d.workspace_bytes = 1 << 24, need - 1
    assert _fwd(L, d) == D.DFA_ERR_CAPACITY
    assert f"{need - 1} given" in dfa_lib.dfa_last_error()
    d.workspace, d.workspace_bytes = (1 << 24) + 8, need
    assert _fwd(L, d) == D.DFA_ERR_INVALID                        # misaligned workspace
    assert "aligned" in dfa_lib.dfa_last_error()
    g = D.make_desc(1, 64, 8, 128, 32768, 1024, 15 * 32768, 0)   # splits: needs scratch
    need_b = dfa_lib.dfa_attn_workspace_size(g, D.DFA_OP_BWD)
    g.workspace, g.workspace_bytes = 1 << 24, need_b - 16

    def bwd(desc):
        return L.dfa_attn_bwd(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                              FAKE, FAKE, FAKE, None)

    assert bwd(g) == D.DFA_ERR_CAPACITY
    assert f"{need_b} bytes required" in dfa_lib.dfa_last_error()


def test_bwd_without_keys_still_computes_delta(dfa_lib):
    """A pair with no keys adds nothing to dq, dk, dv, but with
    compute_delta = 1 it still writes delta, which later pairs of the query
    chunk read: without a GPU the delta launch is attempted (DFA_ERR_HIP),
    and with compute_delta = 0 the call returns at once."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present (the GPU tests cover this case)")
    L = dfa_lib.lib()
    d = D.make_desc(1, 2, 2, 64, 64, 0)

    def bwd(cd):
        return L.dfa_attn_bwd(ctypes.byref(d), None, None, None, FAKE, None, FAKE, FAKE, cd,
                              None, None, None, None)

    assert bwd(0) == D.DFA_OK
    assert bwd(1) == D.DFA_ERR_HIP


def test_chunk_transfer_argument_errors(dfa_lib):
    """The emulated exchange copy checks its arguments before the runtime:
    negative sizes, null pointers and overlapping ranges are rejected, and a
    zero-byte transfer enqueues nothing."""
    L = dfa_lib.lib()
    a, b = ctypes.c_void_p(1 << 24), ctypes.c_void_p((1 << 24) + 4096)
    assert L.dfa_chunk_transfer(a, b, -1, None) == D.DFA_ERR_INVALID
    assert L.dfa_chunk_transfer(None, b, 16, None) == D.DFA_ERR_INVALID
    assert L.dfa_chunk_transfer(a, None, 16, None) == D.DFA_ERR_INVALID
    assert L.dfa_chunk_transfer(a, b, 4097, None) == D.DFA_ERR_INVALID    # ranges overlap
    assert "overlap" in dfa_lib.dfa_last_error()
    assert L.dfa_chunk_transfer(b, a, 4097, None) == D.DFA_ERR_INVALID
    assert L.dfa_chunk_transfer(None, None, 0, None) == D.DFA_OK


def _visible_keys(lq, lk, q0, k0, causal, win, r):
    """Keys of the chunk that local query row r sees (written out plainly)."""
    q = q0 + r
    hi = k0 + lk - 1 if not causal else min(k0 + lk - 1, q)
    lo = k0 if win <= 0 else max(k0, q - win + 1)
    return max(0, hi - lo + 1)


def test_work_order_follows_the_longest_work(dfa_lib):
    """Host: the forward and dQ take row tiles first to last exactly when the
    pair's first row sees more keys than its last; dK/dV takes its 256-key
    blocks last to first exactly when its last block has more query-row steps
    than its first (32-row steps from the block's first visible row)."""
    cases = [  # (lq, lk, q0, k0, causal, win)
        (1024, 1024, 0, 0, True, 0),          # diagonal
        (1024, 1024, 4096, 0, True, 0),       # fully visible
        (1024, 1024, 0, 0, False, 0),         # non-causal
        (1024, 1024, 0, 0, True, 300),        # windowed diagonal
        (1024, 1024, 1024, 0, True, 512),     # band pair: the window leaves the key chunk
        (1024, 1024, 1024, 0, True, 2048),    # band pair the window still covers
        (1000, 700, 900, 0, True, 400),       # ragged band pair
        (512, 1536, 1024, 0, True, 0),        # rows starting inside the key chunk
        (0, 256, 0, 0, True, 0), (256, 0, 0, 0, True, 0),
    ]
    seen_rows = seen_keys = 0
    for lq, lk, q0, k0, causal, win in cases:
        d = D.make_desc(1, 8, 2, 128, lq, lk, q0, k0, causal, window=win)
        rows_up, keys_down = D.dfa_test_work_order(d)
        if lq == 0 or lk == 0:
            assert (rows_up, keys_down) == (False, False)
            continue
        want_rows = (_visible_keys(lq, lk, q0, k0, causal, win, 0) >
                     _visible_keys(lq, lk, q0, k0, causal, win, lq - 1))
        assert rows_up == want_rows, (lq, lk, q0, k0, causal, win)

        def steps(j_lo):  # row steps of the key block starting at key j_lo
            first = None
            last = -1
            for r in range(lq):
                q = q0 + r
                if any((not causal or k0 + j <= q) and (win <= 0 or q - (k0 + j) < win)
                       for j in range(j_lo, min(j_lo + 256, lk))):
                    first = r if first is None else first
                    last = r
            return 0 if first is None else (last // 32) - (first // 32) + 1
        last_block = (lk - 1) // 256 * 256
        assert keys_down == (steps(last_block) > steps(0)), (lq, lk, q0, k0, causal, win)
        seen_rows += rows_up
        seen_keys += keys_down
    assert seen_rows >= 2 and seen_keys >= 2  # both orders are exercised
    L = dfa_lib.lib()
    c = ctypes.c_int32(0)
    d = D.make_desc(1, 8, 2, 128, 256, 256)
    assert L.dfa_test_work_order(ctypes.byref(d), None, ctypes.byref(c)) == D.DFA_ERR_INVALID
    assert L.dfa_test_work_order(None, ctypes.byref(c), ctypes.byref(c)) == D.DFA_ERR_INVALID
