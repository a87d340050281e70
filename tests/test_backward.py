"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the CPU
float64 oracle (oracle.attention_bwd_ref).

The forward kernel produces O and LSE, fa_bwd the gradients; each element of
dQ, dK, dV is compared with the oracle's gradient under the elementwise bound
derived in tests/bwd_tolerance.py from the kernel's bf16 roundings.  Small
cases span several 128-row / 128-key tiles with ragged tails and cover MHA,
GQA, MQA, both head dims, Lq != Lk (rows that see no key, keys no row sees),
causal, sliding and two-sided windows.  The causal MHA workload runs at full
size with sampled rows and keys, and two runs must agree bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from bwd_tolerance import bwd_tolerance, key_rows_tolerance, query_rows_tolerance, ratio
from gpu_helpers import bits, dev, f64

pytestmark = pytest.mark.gpu


def make_case(seed, B, Lq, Lk, Hq, Hkv, d, causal, window):
    w = workloads.random_dense(seed, B, Lq, Lk, Hq, Hkv, d, causal, window)
    return w, workloads.upstream_grad(seed + 7919, (B, Lq, Hq, d))


def run_bwd(fa, w, dout):
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o, lse = fa.fa_fwd(q, k, v, w.scale, w.causal, w.window)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, dev(dout), w.scale, w.causal, w.window)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


BWD_CASES = [
    # B, Lq, Lk, Hq, Hkv, d, causal, window
    (2, 200, 200, 4, 2, 128, True, (-1, -1)),
    (1, 300, 300, 2, 1, 64, True, (50, 0)),
    (2, 130, 257, 4, 4, 128, False, (-1, -1)),
    (1, 257, 130, 3, 1, 64, True, (-1, -1)),       # Lq > Lk: the first 127 rows see nothing
    (1, 64, 64, 8, 2, 128, False, (20, 20)),
    (1, 1, 300, 2, 1, 128, True, (-1, -1)),       # one query row
    (1, 513, 513, 2, 2, 128, True, (-1, -1)),
    (1, 100, 400, 4, 1, 128, False, (30, 10)),    # keys no row sees
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c[:6])) + f"-c{int(c[6])}-w{c[7][0]}_{c[7][1]}")
def test_bwd_sweep(fa, case):
    w, dout = make_case(400 + sum(case[:6]), *case)
    got = run_bwd(fa, w, dout)
    qb, kb, vb, db = bits(w.q), bits(w.k), bits(w.v), bits(dout)
    ref = oracle.attention_bwd_ref(qb, kb, vb, db, w.scale, w.causal, w.window)
    tol = bwd_tolerance(qb, kb, vb, db, w.scale, w.causal, w.window, ref)
    for name, g, r, t in zip(("dq", "dk", "dv"), got, ref, tol):
        g = f64(g)
        assert np.isfinite(g).all(), name
        x = ratio(g, r, t)
        print(f"[parity] bwd{case} {name}: max err/tol {x:.3f}", flush=True)
        assert x <= 1.0, name


def test_bwd_full_causal_mha_sampled_and_deterministic(fa):
    w = workloads.causal_mha()
    B, L, H, d = w.q.shape
    dout = workloads.upstream_grad(1002, (B, L, H, d))
    dq, dk, dv = run_bwd(fa, w, dout)
    dq2, dk2, dv2 = run_bwd(fa, w, dout)
    for a, b2 in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b2.view(torch.int16))     # bitwise reproducible
    qb, kb, vb, db = bits(w.q), bits(w.k), bits(w.v), bits(dout)
    rng = np.random.default_rng(12)
    fixed = [0, 1, 63, 64, 127, 128, 1023, 2046, 2047]
    for b, h in [(0, 0), (1, 17), (3, 31)]:
        rows = np.unique(np.concatenate([fixed, rng.integers(0, L, 8)]))
        ref = oracle.attention_bwd_query_rows_ref(qb, kb, vb, db, b, h, rows, w.scale, True)
        tol = query_rows_tolerance(qb, kb, vb, db, b, h, rows, w.scale, True, (-1, -1), ref)
        x = ratio(f64(dq[b, rows, h]), ref, tol)
        print(f"[parity] bwd full dq b{b} h{h}: max err/tol {x:.3f}", flush=True)
        assert x <= 1.0
    for b, g in [(0, 5), (2, 30)]:
        keys = np.unique(np.concatenate([fixed, rng.integers(0, L, 8)]))
        rk, rv = oracle.attention_bwd_key_rows_ref(qb, kb, vb, db, b, g, keys, w.scale, True)
        tk, tv = key_rows_tolerance(qb, kb, vb, db, b, g, keys, w.scale, True, (-1, -1), rk, rv)
        xk = ratio(f64(dk[b, keys, g]), rk, tk)
        xv = ratio(f64(dv[b, keys, g]), rv, tv)
        print(f"[parity] bwd full dk/dv b{b} g{g}: max err/tol {xk:.3f} / {xv:.3f}", flush=True)
        assert xk <= 1.0 and xv <= 1.0


def test_bwd_huge_window_equals_unbounded(fa):
    w, dout = make_case(77, 1, 150, 200, 4, 2, 128, True, (-1, -1))
    q, k, v, do = dev(w.q), dev(w.k), dev(w.v), dev(dout)
    o, lse = fa.fa_fwd(q, k, v, w.scale, True)
    a = fa.fa_bwd(q, k, v, o, lse, do, w.scale, True, (2 ** 31 - 1, 2 ** 31 - 1))
    b = fa.fa_bwd(q, k, v, o, lse, do, w.scale, True, (-1, -1))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_full_causal_gqa_long_sampled(fa):
    """The long-context GQA workload as bench.py times it (B=1, Hq=32, Hkv=8,
    L=16384): dQ on sampled rows; dK, dV on sampled keys of the second half
    (rows before a key never see it under the causal mask, so only rows from
    the earliest sampled key on are summed)."""
    w = workloads.causal_gqa_long()
    B, L, Hq, d = w.q.shape
    dout = workloads.upstream_grad(1003, (B, L, Hq, d))
    dq, dk, dv = run_bwd(fa, w, dout)
    qb, kb, vb, db = bits(w.q), bits(w.k), bits(w.v), bits(dout)
    rng = np.random.default_rng(13)
    for h in (0, 3, 29):
        rows = np.unique(np.concatenate([[0, 127, 128, 8191, 16383], rng.integers(0, L, 4)]))
        ref = oracle.attention_bwd_query_rows_ref(qb, kb, vb, db, 0, h, rows, w.scale, True)
        tol = query_rows_tolerance(qb, kb, vb, db, 0, h, rows, w.scale, True, (-1, -1), ref)
        x = ratio(f64(dq[0, rows, h]), ref, tol)
        print(f"[parity] bwd gqa-long dq h{h}: max err/tol {x:.3f}", flush=True)
        assert x <= 1.0
    for g in (0, 7):
        keys = np.unique(np.concatenate([[14336, 15999, 16256, 16383], rng.integers(14336, L, 4)]))
        start = int(keys.min())
        rk, rv = oracle.attention_bwd_key_rows_ref(qb, kb, vb, db, 0, g, keys, w.scale, True,
                                                   row_start=start)
        tk, tv = key_rows_tolerance(qb, kb, vb, db, 0, g, keys, w.scale, True, (-1, -1), rk, rv,
                                    row_start=start)
        xk, xv = ratio(f64(dk[0, keys, g]), rk, tk), ratio(f64(dv[0, keys, g]), rv, tv)
        print(f"[parity] bwd gqa-long dk/dv g{g}: max err/tol {xk:.3f} / {xv:.3f}", flush=True)
        assert xk <= 1.0 and xv <= 1.0


# ------------------------------------------------------------------ varlen
VARLEN_BWD_CASES = [
    # lens_q, lens_k (None: same), Hq, Hkv, d, causal, window
    ([1, 0, 7, 128, 129, 300], None, 4, 2, 128, True, (-1, -1)),
    ([250, 3, 64], None, 2, 1, 64, False, (-1, -1)),
    ([513, 17], None, 8, 8, 128, False, (30, 30)),
    ([100, 0, 260], [300, 50, 260], 4, 2, 128, True, (-1, -1)),    # Lk != Lq; no rows
    ([300, 40], [0, 400], 4, 1, 64, True, (64, -1)),               # a sequence without keys
]


@pytest.mark.parametrize("case", VARLEN_BWD_CASES, ids=lambda c: f"n{len(c[0])}-h{c[2]}-kv{c[3]}-d{c[4]}-c{int(c[5])}-w{c[6][0]}")
def test_bwd_varlen_sweep(fa, case):
    lq, lk, Hq, Hkv, d, causal, window = case
    lk = lq if lk is None else lk
    seed = 600 + sum(lq) + d
    q, k, v, cq, ck = workloads.random_varlen_qk(seed, lq, lk, Hq, Hkv, d)
    dout = workloads.upstream_grad(seed + 1, tuple(q.shape))
    scale = 1.0 / np.sqrt(d)
    cqd, ckd = dev(torch.from_numpy(cq)), dev(torch.from_numpy(ck))
    mq, mk = max(lq), max(lk)
    qd, kd, vd = dev(q), dev(k), dev(v)
    o, lse = fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, mq, mk, scale, causal, window)
    got = fa.fa_bwd_varlen(qd, kd, vd, o, lse, dev(dout), cqd, ckd, mq, mk, scale, causal, window)
    torch.cuda.synchronize()
    qb, kb, vb, db = bits(q), bits(k), bits(v), bits(dout)
    ref = oracle.attention_varlen_bwd_ref(qb, kb, vb, db, cq, ck, scale, causal, window)
    # tolerance per sequence (the bound of the dense case on each sequence's slices)
    tol = [np.full_like(r, 1e-5) for r in ref]
    for b in range(len(lq)):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        if lq[b] == 0 or lk[b] == 0:
            continue
        rb = tuple(x[None] for x in (ref[0][qs], ref[1][ks], ref[2][ks]))
        tb = bwd_tolerance(qb[None, qs], kb[None, ks], vb[None, ks], db[None, qs], scale, causal,
                           window, rb)
        tol[0][qs], tol[1][ks], tol[2][ks] = tb[0][0], tb[1][0], tb[2][0]
    for name, g, r, t in zip(("dq", "dk", "dv"), got, ref, tol):
        g = f64(g.cpu())
        assert np.isfinite(g).all(), name
        x = ratio(g, r, t)
        print(f"[parity] bwd varlen{case} {name}: max err/tol {x:.3f}", flush=True)
        assert x <= 1.0, name
