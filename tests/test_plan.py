"""Host plans of the plan/run split (fa_varlen_plan, fa_decode_plan), checked on
the CPU.

The plan must list every query tile of every sequence exactly once, and list
them by non-increasing cost, where the cost of a tile is the number of 64-key
tiles the kernel visits for its 128 query rows.  The cost here is derived by
brute force from the oracle's visibility matrix (the union of the keys any row
of the tile can see, counted in 64-key tiles; for causal and sliding-window
masks that union is one interval, which is the range the kernel walks), not
from the library's formula.

The decode plan must list exactly the (request, split) pairs whose key range
holds a key the new token sees, ordered by that key count, heaviest first;
again derived by brute force from the oracle's visibility of a one-row query.
"""

import ctypes
import os

import numpy as np
import pytest

import exact_attention_17_amd as fa
import oracle
from exact_attention_17_amd import build

OK, INVALID, WORKSPACE = 0, 1, 3
BM, BN = 128, 64


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    return fa.load_library()


def cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def brute_cost(lq, lk, qt, causal, window):
    rows = np.arange(qt * BM, min(qt * BM + BM, lq))
    vis = oracle.key_visibility(lq, lk, causal, window[0], window[1], rows=rows)
    keys = np.nonzero(vis.any(axis=0))[0]
    if keys.size:                       # the visible keys of a tile form one interval
        assert keys[-1] - keys[0] + 1 == keys.size
    return len(np.unique(keys // BN))


def check_plan(plan, lq_list, lk_list, causal, window):
    items = [(b, t) for b, L in enumerate(lq_list) for t in range(-(-L // BM))]
    got = [tuple(x) for x in plan.tolist()]
    assert sorted(got) == sorted(items)                      # every tile exactly once
    cost = [brute_cost(lq_list[b], lk_list[b], t, causal, window) for b, t in got]
    assert all(cost[i] >= cost[i + 1] for i in range(len(cost) - 1))   # heaviest first
    # equal costs keep sequence order, and within a sequence the later tile first
    for i in range(len(got) - 1):
        if cost[i] == cost[i + 1]:
            (b0, t0), (b1, t1) = got[i], got[i + 1]
            assert b0 < b1 or (b0 == b1 and t0 > t1)
    return cost


CASES = [
    ([1, 0, 7, 128, 129, 300], None, True, (-1, -1)),
    ([1, 0, 7, 128, 129, 300], None, True, (50, 0)),
    ([250, 3, 64], None, False, (-1, -1)),
    ([513, 17], None, False, (30, 30)),
    ([100, 700, 260], [900, 700, 1000], True, (-1, -1)),     # Lk > Lq: bottom-right causal
    ([300, 40], [50, 400], True, (64, -1)),                  # Lk < Lq: leading rows see nothing
    ([1000, 2000, 64, 1500], None, True, (256, 0)),
    ([0, 0, 5], [0, 9, 0], False, (-1, -1)),                 # empty keys give cost 0
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{len(c[0])}-c{int(c[2])}-w{c[3][0]}_{c[3][1]}")
def test_plan_lists_every_tile_heaviest_first(case):
    lq, lk, causal, window = case
    lk = lq if lk is None else lk
    plan = fa.fa_varlen_plan(cu(lq), cu(lk), causal, window)
    assert plan.dtype == np.int32 and plan.shape == (sum(-(-L // BM) for L in lq), 2)
    check_plan(plan, lq, lk, causal, window)


def test_plan_of_a_skewed_batch():
    # the full-size varlen + window batch's length mix: long sequences first
    import workloads
    lens = [int(x) for x in workloads.varlen_window_lengths()]
    plan = fa.fa_varlen_plan(cu(lens), cu(lens), True, (4096, 0))
    cost = check_plan(plan, lens, lens, True, (4096, 0))
    # a tile deep in a long sequence sees 4096 + 128 keys starting on a
    # 64-key boundary (Lq = Lk): 66 key tiles; the first tile of a sequence 2
    assert cost[0] == 66 and cost[-1] == 2
    # without a window the last tile of the longest sequence comes first
    plan = fa.fa_varlen_plan(cu(lens), cu(lens), True, (-1, -1))
    b = int(np.argmax(lens))
    assert tuple(plan[0]) == (b, -(-lens[b] // BM) - 1)


def test_plan_empty_and_counting(lib):
    assert fa.fa_varlen_plan([0, 0, 0], [0, 3, 8], True).shape == (0, 2)
    n = ctypes.c_int(-1)
    c = cu([300, 5])
    ptr = c.ctypes.data_as(ctypes.c_void_p)
    assert lib.fa_varlen_plan(ptr, ptr, 2, 1, -1, -1, None, 0, ctypes.byref(n)) == OK
    assert n.value == 4
    buf = np.full(8, -7, dtype=np.int32)
    n.value = -1
    # too small a buffer: the count is still reported and the buffer is untouched
    assert lib.fa_varlen_plan(ptr, ptr, 2, 1, -1, -1, buf.ctypes.data_as(ctypes.c_void_p), 3,
                              ctypes.byref(n)) == WORKSPACE
    assert n.value == 4 and (buf == -7).all()


@pytest.mark.parametrize("cq,ck,kw", [
    ([1, 5], [0, 5], {}),                 # cu[0] != 0
    ([0, 5, 3], [0, 5, 6], {}),           # decreasing
    ([0, 5], [0, -1], {}),
    ([0, 5], [0, 5], dict(causal=2)),
    ([0, 5], [0, 5], dict(wl=-2)),
    ([0, 5], [0, 5], dict(B=0)),
])
def test_plan_rejects(lib, cq, ck, kw):
    a = dict(B=len(cq) - 1, causal=1, wl=-1, wr=-1)
    a.update(kw)
    cq = np.asarray(cq, dtype=np.int32)
    ck = np.asarray(ck, dtype=np.int32)
    n = ctypes.c_int(0)
    buf = np.zeros(16, dtype=np.int32)
    st = lib.fa_varlen_plan(cq.ctypes.data_as(ctypes.c_void_p), ck.ctypes.data_as(ctypes.c_void_p),
                            a["B"], a["causal"], a["wl"], a["wr"],
                            buf.ctypes.data_as(ctypes.c_void_p), 8, ctypes.byref(n))
    assert st == INVALID
    assert lib.fa_varlen_plan(None, None, 1, 1, -1, -1, None, 0, ctypes.byref(n)) == INVALID


# ------------------------------------------------------------------ decode
def decode_items(lens, split, window_left):
    """(b, s) -> visible key count, by brute force over each request's keys."""
    out = {}
    for b, L in enumerate(lens):
        if L == 0:
            continue
        vis = oracle.key_visibility(1, L, True, window_left, -1)[0]
        for s, n in enumerate(np.add.reduceat(vis.astype(np.int64), np.arange(0, L, split))):
            if n:
                out[(b, s)] = int(n)
    return out


DECODE_PLAN_CASES = [
    ([1, 15, 16, 17, 511, 512, 513, 1000], 16, 64, 512, -1),
    ([1, 15, 16, 17, 511, 512, 513, 1000], 16, 64, 16, -1),
    ([300, 64, 900], 16, 60, 0, -1),
    ([1000, 50], 16, 64, 512, 100),
    ([1000, 50, 513], 1, 1024, 128, 600),
    ([0, 40, 0], 16, 8, 512, -1),
    ([0, 0], 16, 8, 512, -1),
]


@pytest.mark.parametrize("case", DECODE_PLAN_CASES,
                         ids=lambda c: f"n{len(c[0])}-p{c[1]}-s{c[3]}-w{c[4]}")
def test_decode_plan_lists_active_splits_heaviest_first(case):
    lens, ps, mb, split, wl = case
    plan = fa.fa_decode_plan(lens, ps, mb, wl, split)
    want = decode_items(lens, split or 512, wl)
    got = [tuple(x) for x in plan.tolist()]
    assert plan.dtype == np.int32 and sorted(got) == sorted(want)
    cost = [want[x] for x in got]
    assert all(cost[i] >= cost[i + 1] for i in range(len(cost) - 1))
    for i in range(len(got) - 1):
        if cost[i] == cost[i + 1]:
            assert got[i] < got[i + 1]          # ties keep (request, split) order


def test_decode_plan_of_the_paged_decode_workload():
    import workloads
    lens, table, _, _ = workloads.paged_decode_layout()
    plan = fa.fa_decode_plan(lens, 16, table.shape[1], -1, 512)
    want = decode_items([int(x) for x in lens], 512, -1)
    assert len(plan) == len(want) == sum(-(-int(L) // 512) for L in lens)
    # full 512-key splits first, then the tails, longest first
    full = sum(int(L) // 512 for L in lens)
    assert all(want[tuple(x)] == 512 for x in plan[:full].tolist())


@pytest.mark.parametrize("lens,kw", [
    ([5, -1], {}), ([129], dict(mb=8)), ([5], dict(split=24)), ([5], dict(split=-16)),
    ([5], dict(wl=-2)), ([5], dict(ps=0)), ([5], dict(mb=0)), ([], {}),
])
def test_decode_plan_rejects(lib, lens, kw):
    a = dict(ps=16, mb=8, wl=-1, split=0)
    a.update(kw)
    sl = np.asarray(lens + [0], dtype=np.int32)
    n = ctypes.c_int(0)
    buf = np.zeros(64, dtype=np.int32)
    st = lib.fa_decode_plan(sl.ctypes.data_as(ctypes.c_void_p), len(lens), a["ps"], a["mb"],
                            a["wl"], a["split"], buf.ctypes.data_as(ctypes.c_void_p), 32,
                            ctypes.byref(n))
    assert st == INVALID


def test_decode_plan_counting(lib):
    sl = np.asarray([1000, 3], dtype=np.int32)
    n = ctypes.c_int(-1)
    p = sl.ctypes.data_as(ctypes.c_void_p)
    assert lib.fa_decode_plan(p, 2, 16, 64, -1, 512, None, 0, ctypes.byref(n)) == OK
    assert n.value == 3
    buf = np.full(4, -7, dtype=np.int32)
    assert lib.fa_decode_plan(p, 2, 16, 64, -1, 512, buf.ctypes.data_as(ctypes.c_void_p), 2,
                              ctypes.byref(n)) == WORKSPACE
    assert n.value == 3 and (buf == -7).all()
