"""bgtq_logquant_plan (host C ABI, no GPU) against the LogQuant selection oracle: replaying the
plans on a simulated high-precision store keeps exactly the oracle's positions at every step,
the leaving rows come out in the oracle's order, and the compaction is conflict-free."""
import ctypes as C
import os

import numpy as np
import pytest

import packed_cache_decode_block_amd as P
from oracle import logquant as lq
from packed_cache_decode_block_amd import _lib, build_lib


@pytest.fixture(scope="module")
def plan_lib():
    """The library's planner, or (BGTQ_SANITIZED_MOCK=1) the AddressSanitizer / UBSan build of the
    host code, which tests/test_sanitized_host.py runs this module against."""
    if os.environ.get("BGTQ_SANITIZED_MOCK") == "1":
        return _lib.bind(build_lib.build_mock(sanitize=True), optional=("bgtq_decode_attention_noalloc",))
    return P.lib


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8, 32])
def test_plans_replay_to_the_oracle(W, plan_lib):
    pl = P.LogQuantPlanner(W, library=plan_lib)
    store = np.full(3 * W, -1, np.int64)        # the simulated store: token position per slot
    left = []
    n = 30 * W + 5
    for p in range(n):
        evict, moves, slot = pl.append(p)
        left += [int(store[s]) for s in evict]                 # rows read before any move
        vacated = set(int(s) for s in evict)
        dsts = [d for _, d in moves]
        assert len(set(dsts)) == len(dsts) and not {s for s, _ in moves} & set(dsts)   # no move reads a written slot
        assert set(dsts) <= vacated and all(d < 2 * W <= s for s, d in moves)
        for s, d in moves:
            store[d] = store[s]
        store[slot] = p
        assert pl.n_hp <= 3 * W and slot == pl.n_hp - 1
        live = store[:pl.n_hp]
        np.testing.assert_array_equal(np.sort(live), lq.select(p + 1, W)[0])
        np.testing.assert_array_equal(live, pl.hp_pos[:pl.n_hp])
    assert left == lq.select(n, W)[1]


def test_plan_errors_change_nothing(plan_lib):
    W = 2
    hp = np.array([0, 1, 2, 3, 4, 5], np.int64)
    n = C.c_int(6)
    ev, ms, md = (np.zeros(W, np.int32) for _ in range(3))
    nm, ns = C.c_int(0), C.c_int(0)
    p64, p32 = C.POINTER(C.c_int64), C.POINTER(C.c_int32)
    call = lambda W_, pos, n_=n: plan_lib.bgtq_logquant_plan(W_, hp.ctypes.data_as(p64), C.byref(n_), pos,
                                                          ev.ctypes.data_as(p32), ms.ctypes.data_as(p32),
                                                          md.ctypes.data_as(p32), C.byref(nm), C.byref(ns))
    assert call(W, 5) == P.E_INVALID                           # not above the held positions
    assert call(0, 9) == P.E_INVALID                           # W < 1
    assert call(W, 9, C.c_int(7)) == P.E_INVALID               # more rows than the 3W ceiling
    hp[3] = 2
    assert call(W, 9) == P.E_INVALID                           # a repeated position
    hp[3] = 3
    assert n.value == 6 and list(hp) == [0, 1, 2, 3, 4, 5]
    assert call(W, 9) == W and n.value == 2 * W + 1            # then a valid call: two rows leave
