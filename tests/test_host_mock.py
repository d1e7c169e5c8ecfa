"""Host logic of the C ABI without a GPU: the real bgtq_host.cpp linked against mock launchers
that check every kernel argument block (pointers set, ranges consistent) and record launches."""
import ctypes as C
import os

import numpy as np
import pytest

from packed_cache_decode_block_amd import _lib, build_lib

FAKE = 0x7F0000000000  # never dereferenced: the mocks only inspect argument blocks


@pytest.fixture(scope="module")
def mock():
    # BGTQ_SANITIZED_MOCK=1: the AddressSanitizer / UBSan build (tests/test_sanitized_host.py runs
    # this module that way, in a process that preloads the ASan runtime)
    san = os.environ.get("BGTQ_SANITIZED_MOCK") == "1"
    lib = _lib.bind(build_lib.build_mock(sanitize=san), optional=("bgtq_decode_attention_noalloc",))
    lib.bgtq_mock_log.restype = C.c_char_p
    lib.bgtq_mock_last_copy.restype = C.c_int64
    lib.bgtq_mock_last_copy.argtypes = [C.c_void_p, C.c_int64]
    return lib


def _desc(nt, **kw):
    d = _lib.CacheDesc()
    base = dict(L=2, B=2, Hq=16, Hkv=2, d=128, n_cap=4096, k_mode=0, budget_units=192, k_bits=4, k_group=32,
                v_mode=0, v_bits=3, n_recent=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    ptrs = ["k_codes", "v_codes", "k_scale", "v_scale", "bits", "sigma", "inv_sigma"]
    if base["k_mode"] == 1:
        ptrs.append("k_zero")
    else:
        ptrs.append("plan")
    if base["v_mode"] == 1:
        ptrs.append("v_zero")
    if base["n_recent"]:
        ptrs += ["recent_k", "recent_v"]
    for i, name in enumerate(ptrs):
        setattr(d, name, FAKE + i * 0x1000000)
    d.n_tokens = nt.ctypes.data_as(C.POINTER(C.c_int64))
    return d


def _call_ok(mock, rc):
    log = mock.bgtq_mock_log().decode()
    assert rc == 0 and "BAD" not in log, (rc, mock.bgtq_last_error(), log)
    return log


FORMATS = [dict(), dict(budget_units=128, v_bits=2), dict(k_mode=1, k_bits=4, k_group=32, v_mode=1, v_bits=2),
           dict(budget_units=192, v_bits=2, n_recent=256), dict(budget_units=256, v_bits=4, Hq=8, Hkv=8),
           dict(k_mode=1, k_group=128, v_bits=4, Hq=4, Hkv=2, n_recent=64),
           dict(budget_units=128, v_bits=2, n_recent=600), dict(Hq=2, Hkv=2, v_bits=2, n_recent=100)]


@pytest.mark.parametrize("fmt", range(len(FORMATS)))
def test_append_then_decode_arguments(mock, fmt):
    nt = np.zeros((2, 2), np.int64)
    d = _desc(nt, **FORMATS[fmt])
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    for n_new in (1, 63, 64, 200, 1000):
        mock.bgtq_mock_reset()
        _call_ok(mock, mock.bgtq_quantize_append(C.byref(d), 1, q, q, 2, n_new, None, None))
        for ns in (0, 1, 3, 40):
            mock.bgtq_mock_reset()
            need = mock.bgtq_decode_workspace_bytes(C.byref(d), ns)
            assert need > 0
            log = _call_ok(mock, mock.bgtq_decode_attention(C.byref(d), 1, q, 2, q, ws, need, ns, None))
            assert log.count("decode") == 1 and log.count("combine") == 1
            # a window of at most 512 rows is attended by the merge itself; a longer one has a
            # split-K launch of its own
            assert log.count("fp16") == (1 if d.n_recent > 512 else 0)
            assert log.count("combine_window") == (1 if 0 < d.n_recent <= 512 else 0)
    assert (nt[1] == 1 + 63 + 64 + 200 + 1000).all() and (nt[0] == 0).all()


def test_ring_eviction_plan(mock):
    """With a 256-token fp16 window, appends quantize exactly the tokens that leave the window."""
    nt = np.zeros((1, 1), np.int64)
    d = _desc(nt, L=1, B=1, n_recent=256, budget_units=192, v_bits=2)
    q = C.c_void_p(FAKE + 0x50000000)
    mock.bgtq_mock_reset()
    _call_ok(mock, mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 100, None, None))
    assert "quant" not in mock.bgtq_mock_log().decode()          # everything still fits the ring
    mock.bgtq_mock_reset()
    _call_ok(mock, mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 300, None, None))
    log = mock.bgtq_mock_log().decode()
    assert "quant" in log and "ring" in log
    assert nt[0, 0] == 400


def test_window_partials_in_the_workspace(mock):
    """A window the merge attends to needs no partial of its own; a longer window's launch needs
    one more per query head."""
    nt = np.zeros((2, 2), np.int64)
    per_part = 2 * 16 * 132 * 4
    for ns in (0, 1, 7):
        base = mock.bgtq_decode_workspace_bytes(C.byref(_desc(nt)), ns)
        assert mock.bgtq_decode_workspace_bytes(C.byref(_desc(nt, n_recent=512)), ns) == base
        assert mock.bgtq_decode_workspace_bytes(C.byref(_desc(nt, n_recent=513)), ns) == base + per_part


def test_capacity_and_failure_leave_state(mock):
    nt = np.zeros((2, 2), np.int64)
    d = _desc(nt, n_cap=128)
    q = C.c_void_p(FAKE + 0x50000000)
    assert mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 129, None, None) == _lib.E_CAPACITY
    assert (nt == 0).all()
    _call_ok(mock, mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 128, None, None))
    assert mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 1, None, None) == _lib.E_CAPACITY
    assert (nt[0] == 128).all()


def test_fp16_comparator_arguments(mock):
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    for (N, B, Hq, Hkv, ns) in ((1, 1, 1, 1, 0), (3000, 2, 16, 2, 5), (131072, 1, 16, 2, 0), (777, 3, 32, 8, 0)):
        mock.bgtq_mock_reset()
        need = mock.bgtq_fp16_decode_workspace_bytes(N, B, Hq, Hkv, ns)
        _call_ok(mock, mock.bgtq_fp16_decode_attention(q, q, N, B, Hq, Hkv, 128, q, 2, q, ws, need, ns, None))
        assert mock.bgtq_mock_launches() == 2


@pytest.mark.parametrize("fmt", range(len(FORMATS)))
def test_decode_step_appends_then_attends(mock, fmt):
    """The combined step matches the lengths that the two separate calls leave.  One token per
    sequence on the plan-driven kernel without an fp16 window is written by the decode launch itself
    (one decode launch and the merge); otherwise the append's launches come before the attention's."""
    nt = np.zeros((2, 2), np.int64)
    f = FORMATS[fmt]
    d = _desc(nt, **f)
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    need = mock.bgtq_decode_workspace_bytes(C.byref(d), 0)
    fusable = f.get("k_mode", 0) == 0 and f.get("Hq", 16) // f.get("Hkv", 2) >= 4 and not f.get("n_recent", 0)
    total = 0
    for n_new in (1, 1, 63, 200, 1):
        mock.bgtq_mock_reset()
        log = _call_ok(mock, mock.bgtq_decode_step(C.byref(d), 1, q, q, q, 2, n_new, None, q, ws, need, 0, None))
        total += n_new
        if fusable and n_new == 1:
            assert log.split() == ["decode_gtq_append", "combine"], log
        else:
            assert log.count("decode") == 1 and log.count("combine") == 1 and "append" not in log
            first_decode = log.index("decode")
            for tag in ("quant", "ring"):
                if tag in log:
                    assert log.index(tag) < first_decode, log
            assert "quant" in log or "ring" in log
        assert (nt[1] == total).all() and (nt[0] == 0).all()


def test_decode_step_failure_leaves_state(mock):
    """Errors found in either half come back before anything is enqueued or counted."""
    nt = np.zeros((2, 2), np.int64)
    d = _desc(nt, n_cap=128)
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    need = mock.bgtq_decode_workspace_bytes(C.byref(d), 0)
    step = lambda n_new, ws_bytes, ws_=ws, n_splits=0: mock.bgtq_decode_step(
        C.byref(d), 0, q, q, q, 2, n_new, None, q, ws_, ws_bytes, n_splits, None)
    cases = [(lambda: step(129, need), _lib.E_CAPACITY),          # append half: capacity
             (lambda: step(1, 16), _lib.E_INVALID),               # attention half: workspace too small
             (lambda: step(1, need, C.c_void_p(FAKE + 0x60000010)), _lib.E_INVALID),   # misaligned workspace
             (lambda: step(0, need), _lib.E_INVALID),             # nothing appended to an empty context
             (lambda: step(1, need, ws, 1 << 20), _lib.E_UNSUPPORTED)]                  # too many splits
    for call, code in cases:
        mock.bgtq_mock_reset()
        assert call() == code, mock.bgtq_last_error()
        assert mock.bgtq_mock_launches() == 0
        assert (nt == 0).all()
    mock.bgtq_mock_reset()
    _call_ok(mock, step(5, need))
    assert (nt[0] == 5).all() and (nt[1] == 0).all()
    mock.bgtq_mock_reset()
    _call_ok(mock, step(0, need))                                 # n_new = 0 attends without appending
    assert "quant" not in mock.bgtq_mock_log().decode() and (nt[0] == 5).all()


def test_logquant_append_plan_and_failures(mock):
    """The log-based filter's appends: below the 3W ceiling only the store write; at it, the store
    reorder (a permutation), the quantize of the W leaving rows, then the write; the packed/high-
    precision split follows the oracle's counts; errors change nothing."""
    from oracle import logquant as lq
    W = 4
    nt = np.zeros((1, 2), np.int64)
    d = _desc(nt, L=1, n_recent=3 * W)
    n_hp = np.zeros((1, 2), np.int32)
    d.n_hp = n_hp.ctypes.data_as(C.POINTER(C.c_int32))
    hp = np.zeros((2, 3 * W), np.int64)
    q = C.c_void_p(FAKE + 0x50000000)
    p64 = C.POINTER(C.c_int64)
    for p in range(40):
        mock.bgtq_mock_reset()
        log = _call_ok(mock, mock.bgtq_logquant_append(C.byref(d), 0, q, q, 2, None, hp.ctypes.data_as(p64), None, 0, None))
        steps = [ln for ln in log.splitlines() if ln]
        kept, left = lq.select(p + 1, W)
        thinned = len(left) > len(lq.select(p, W)[1])          # the oracle halved at this token
        assert steps == (["permute", "quant", "ring"] if thinned else ["ring"]), (p, steps)
        assert (nt[0] == p + 1).all() and (n_hp[0] == len(kept)).all()
        assert sorted(hp[0, :n_hp[0, 0]]) == kept
    # the positional-ring entry points refuse a cache under the log-based filter
    assert mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 1, None, None) == _lib.E_INVALID
    # errors: no store positions array, an inconsistent count, capacity; nothing changes
    snap = (nt.copy(), n_hp.copy(), hp.copy())
    assert mock.bgtq_logquant_append(C.byref(d), 0, q, q, 2, None, None, None, 0, None) == _lib.E_INVALID
    n_hp[0, 1] = 3 * W + 1
    assert mock.bgtq_logquant_append(C.byref(d), 0, q, q, 2, None, hp.ctypes.data_as(p64), None, 0, None) == _lib.E_INVALID
    n_hp[0, 1] = snap[1][0, 1]
    d2 = _desc(nt, L=1, n_recent=3 * W, n_cap=64)
    d2.n_hp = d.n_hp
    while n_hp[0, 0] < 3 * W:                                   # fill to the ceiling, then overflow n_cap
        _call_ok(mock, mock.bgtq_logquant_append(C.byref(d2), 0, q, q, 2, None, hp.ctypes.data_as(p64), None, 0, None))
    nt[0] = 100
    pre = (nt.copy(), n_hp.copy(), hp.copy())
    assert mock.bgtq_logquant_append(C.byref(d2), 0, q, q, 2, None, hp.ctypes.data_as(p64), None, 0, None) == _lib.E_CAPACITY
    assert (nt == pre[0]).all() and (n_hp == pre[1]).all() and (hp == pre[2]).all()


def test_prepare_metadata_and_plan_requirement(mock):
    """The Block-GTQ decode needs the layer's plan: bgtq_prepare_metadata launches one plan kernel
    per layer; a descriptor without a plan is refused before any launch; affine keys have none."""
    nt = np.full((2, 2), 500, np.int64)
    d = _desc(nt)
    mock.bgtq_mock_reset()
    _call_ok(mock, mock.bgtq_prepare_metadata(C.byref(d), 1, None))
    assert mock.bgtq_mock_log().decode().split() == ["plan"]
    assert mock.bgtq_prepare_metadata(C.byref(d), 2, None) == _lib.E_INVALID
    assert mock.bgtq_cache_bytes(C.byref(d), _lib.BUF_PLAN) == 2 * 2 * _lib.PLAN_BYTES
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    d.plan = None
    mock.bgtq_mock_reset()
    assert mock.bgtq_decode_attention(C.byref(d), 0, q, 2, q, ws, 1 << 30, 0, None) == _lib.E_INVALID
    assert b"plan" in mock.bgtq_last_error() and mock.bgtq_mock_launches() == 0
    da = _desc(nt, k_mode=1, k_bits=4, k_group=32, v_mode=1, v_bits=2)
    assert mock.bgtq_cache_bytes(C.byref(da), _lib.BUF_PLAN) == 0
    assert mock.bgtq_prepare_metadata(C.byref(da), 0, None) == _lib.E_INVALID


def test_decode_path_routing(mock):
    """decode_path picks the kernel family: Block-GTQ keys at 8 query heads per kv head take the
    plan-driven matrix-core kernel by default and the vector-ALU kernel on the vector path (which
    needs no plan), with workspaces sized for each; other values are refused before any launch."""
    nt = np.full((2, 2), 3000, np.int64)
    d = _desc(nt)
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    need = mock.bgtq_decode_workspace_bytes(C.byref(d), 0)
    mock.bgtq_mock_reset()
    log = _call_ok(mock, mock.bgtq_decode_attention(C.byref(d), 0, q, 2, q, ws, need, 0, None))
    assert log.split() == ["decode_gtq", "combine"], log
    d.decode_path = _lib.DECODE_VECTOR
    d.plan = None
    need_v = mock.bgtq_decode_workspace_bytes(C.byref(d), 0)
    assert need_v > 0
    for ns in (0, 1, 5):
        mock.bgtq_mock_reset()
        log = _call_ok(mock, mock.bgtq_decode_attention(C.byref(d), 0, q, 2, q, ws,
                                                        mock.bgtq_decode_workspace_bytes(C.byref(d), ns), ns, None))
        assert log.split() == ["decode_vector", "combine"], log
    for bad in (2, -1):
        d.decode_path = bad
        mock.bgtq_mock_reset()
        assert mock.bgtq_decode_attention(C.byref(d), 0, q, 2, q, ws, need, 0, None) == _lib.E_INVALID
        assert b"decode_path" in mock.bgtq_last_error() and mock.bgtq_mock_launches() == 0


def test_value_rotation_needs_no_fp16_window(mock):
    """The value rotation is refused, before any launch, with an fp16 window; without one the
    merge gets the layer's sign bits."""
    nt = np.full((2, 2), 300, np.int64)
    d = _desc(nt, budget_units=192, v_bits=2, n_recent=256)
    d.v_rot = FAKE + 0x7000000
    q = C.c_void_p(FAKE + 0x50000000)
    ws = C.c_void_p(FAKE + 0x60000000)
    mock.bgtq_mock_reset()
    assert mock.bgtq_decode_attention(C.byref(d), 0, q, 2, q, ws, 1 << 30, 0, None) == _lib.E_UNSUPPORTED
    assert mock.bgtq_quantize_append(C.byref(d), 0, q, q, 2, 1, None, None) == _lib.E_UNSUPPORTED
    assert mock.bgtq_mock_launches() == 0
    d2 = _desc(nt)
    d2.v_rot = FAKE + 0x7000000
    need = mock.bgtq_decode_workspace_bytes(C.byref(d2), 0)
    mock.bgtq_mock_reset()
    _call_ok(mock, mock.bgtq_decode_attention(C.byref(d2), 1, q, 2, q, ws, need, 0, None))
    # a one-token step with rotated values keeps the separate append launch (the fused path
    # quantizes without the rotation)
    mock.bgtq_mock_reset()
    log = _call_ok(mock, mock.bgtq_decode_step(C.byref(d2), 1, q, q, q, 2, 1, None, q, ws, need, 0, None))
    assert "append" not in log and ("quant" in log), log


def test_logquant_permutation_in_workspace(mock):
    """Above 1536 permutation entries (B * 3W) the store permutation goes through the caller's
    workspace: refused without one, copied there (a valid permutation per sequence) with one."""
    from oracle import logquant as lq
    W = 64
    B = 9                                                          # 9 * 192 = 1728 entries
    nt = np.zeros((1, B), np.int64)
    d = _desc(nt, L=1, B=B, n_recent=3 * W)
    n_hp = np.zeros((1, B), np.int32)
    d.n_hp = n_hp.ctypes.data_as(C.POINTER(C.c_int32))
    hp = np.zeros((B, 3 * W), np.int64)
    q = C.c_void_p(FAKE + 0x50000000)
    p64 = C.POINTER(C.c_int64)
    need = mock.bgtq_logquant_workspace_bytes(C.byref(d), 0)
    assert need >= B * 3 * W * 2 and need % 256 == 0
    ws = C.c_void_p(FAKE + 0x60000000)
    assert mock.bgtq_logquant_append(C.byref(d), 0, q, q, 2, None, hp.ctypes.data_as(p64), None, 0, None) == _lib.E_INVALID
    assert mock.bgtq_logquant_append(C.byref(d), 0, q, q, 2, None, hp.ctypes.data_as(p64), ws, need - 256, None) == _lib.E_INVALID
    assert (nt == 0).all()
    for p in range(3 * W + 1):
        mock.bgtq_mock_reset()
        log = _call_ok(mock, mock.bgtq_logquant_append(C.byref(d), 0, q, q, 2, None, hp.ctypes.data_as(p64), ws, need, None))
    assert log.split() == ["copy", "permute", "quant", "ring"], log
    kept, _ = lq.select(3 * W + 1, W)
    assert (n_hp[0] == len(kept)).all() and all(sorted(hp[b, :len(kept)]) == kept for b in range(B))


def test_logquant_prefill_gathers_the_oracle_selection(mock):
    """The one-call prefill: the gather indices it copies are the oracle's leaving tokens in leaving
    order, then the kept ones; the quantize and the store write read them; the bookkeeping ends as
    n_prompt one-token appends leave it (slot order aside).  Errors change nothing."""
    from oracle import logquant as lq
    W, B, n = 8, 2, 1000
    nt = np.zeros((1, B), np.int64)
    d = _desc(nt, L=1, B=B, n_recent=3 * W, n_cap=1024)
    n_hp = np.zeros((1, B), np.int32)
    d.n_hp = n_hp.ctypes.data_as(C.POINTER(C.c_int32))
    hp = np.zeros((B, 3 * W), np.int64)
    q = C.c_void_p(FAKE + 0x50000000)
    p64 = C.POINTER(C.c_int64)
    ws = C.c_void_p(FAKE + 0x60000000)
    need = mock.bgtq_logquant_workspace_bytes(C.byref(d), n)
    assert need >= (n + 3 * W) * 4
    pre = lambda ws_, nb, n_=n: mock.bgtq_logquant_prefill(C.byref(d), 0, q, q, 2, n_, None, hp.ctypes.data_as(p64),
                                                           ws_, nb, None)
    for call, code in ((lambda: pre(None, 0), _lib.E_INVALID), (lambda: pre(ws, need - 256), _lib.E_INVALID),
                       (lambda: pre(ws, need, 0), _lib.E_INVALID),
                       (lambda: pre(ws, mock.bgtq_logquant_workspace_bytes(C.byref(d), 1100), 1100), _lib.E_CAPACITY)):
        mock.bgtq_mock_reset()
        assert call() == code, mock.bgtq_last_error()
        assert mock.bgtq_mock_launches() == 0 and (nt == 0).all() and (n_hp == 0).all()
    mock.bgtq_mock_reset()
    log = _call_ok(mock, pre(ws, need))
    assert log.split() == ["copy", "quant", "ring"], log
    kept, left = lq.select(n, W)
    idx = np.zeros(len(left) + len(kept), np.int32)
    assert mock.bgtq_mock_last_copy(idx.ctypes.data_as(C.c_void_p), idx.nbytes) == idx.nbytes
    assert list(idx[:len(left)]) == left and list(idx[len(left):]) == kept
    assert (nt[0] == n).all() and (n_hp[0] == len(kept)).all()
    assert all(list(hp[b, :len(kept)]) == kept for b in range(B)) and (hp[:, len(kept):] == -1).all()
    assert pre(ws, need) == _lib.E_INVALID                         # a started layer is refused
