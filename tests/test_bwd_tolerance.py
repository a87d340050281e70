"""The backward tolerance (tests/bwd_tolerance.py) is not vacuous: the float64
oracle rounded once to bf16 passes it, and plausible kernel mistakes -- a key
tile dropped from dQ, a missing delta term, the wrong scale on dK, one row's
contribution lost from dV -- each exceed it (checked on the CPU).  Smaller
ones too: one key missing from dQ, dQ 3% or dK 4% too large."""

import numpy as np

import oracle
from bwd_tolerance import bwd_tolerance, ratio

RNG = np.random.default_rng(99)


def bf16(x):
    a = np.asarray(x, dtype=np.float32).view(np.uint32)
    r = ((a + 0x7FFF + ((a >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def case():
    B, Lq, Lk, Hq, Hkv, d = 1, 96, 160, 4, 2, 32
    q, k, v, do = (bf16(RNG.standard_normal(s)) for s in
                   ((B, Lq, Hq, d), (B, Lk, Hkv, d), (B, Lk, Hkv, d), (B, Lq, Hq, d)))
    return q, k, v, do, 0.3, True, (-1, -1)


def test_tolerance_passes_rounded_oracle_and_catches_mistakes():
    q, k, v, do, scale, causal, window = case()
    ref = oracle.attention_bwd_ref(q, k, v, do, scale, causal, window)
    tol = bwd_tolerance(q, k, v, do, scale, causal, window, ref)
    up = lambda g: (bf16(g).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for g, r, t in zip(ref, ref, tol):
        assert ratio(up(g), r, t) < 0.6

    # mistakes: last 64 keys dropped from dQ; delta term missing; dK without
    # scale; one query row missing from dV
    k_cut = np.array(k)
    k_cut[:, -64:] = 0
    dq_cut = oracle.attention_bwd_ref(q, k_cut, v, do, scale, causal, window)[0]
    assert ratio(dq_cut, ref[0], tol[0]) > 1
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert ratio(ref[1] / scale, ref[1], tol[1]) > 1
    do_cut = np.array(do)
    do_cut[:, 50] = 0
    dv_cut = oracle.attention_bwd_ref(q, k, v, do_cut, scale, causal, window)[2]
    assert ratio(dv_cut, ref[2], tol[2]) > 1
    # a missing delta: dS = P dP, i.e. the gradient with delta forced to 0
    Q = qf[0, :, 0]
    K = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0, :, 0]
    V = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0, :, 0]
    DO = (do.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0, :, 0]
    vis = oracle.key_visibility(96, 160, True)
    _, _, P = oracle.attend_rows(Q, K, V, scale, vis)
    dq_nodelta = scale * (P * (DO @ V.T)) @ K
    assert ratio(dq_nodelta, ref[0][0, :, 0], tol[0][0, :, 0]) > 1


def test_tolerance_catches_small_mistakes():
    """One key's contribution missing from dQ (the last key, seen by the last
    rows only) and a few percent of scale error on dQ or dK."""
    q, k, v, do, scale, causal, window = case()
    ref = oracle.attention_bwd_ref(q, k, v, do, scale, causal, window)
    tol = bwd_tolerance(q, k, v, do, scale, causal, window, ref)
    k_one = np.array(k)
    k_one[:, 150] = 0
    dq_one = oracle.attention_bwd_ref(q, k_one, v, do, scale, causal, window)[0]
    assert ratio(dq_one, ref[0], tol[0]) > 2
    assert ratio(ref[0] * 1.03, ref[0], tol[0]) > 1
    assert ratio(ref[1] * 1.04, ref[1], tol[1]) > 1
