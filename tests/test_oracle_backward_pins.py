"""Pins of the backward oracle (oracle.backward) to facts other than itself.

  * central finite differences of the forward oracle's loss sum(O * dO), which
    is pinned on its own, element by element on tiny cases (every mask mode,
    GQA, Lq != Lk, rows with no visible key);
  * PyTorch autograd in float64 through a plain masked-softmax attention (an
    independent derivation of the chain rule);
  * exact invariants: the keys of a KV head can all move by one vector
    without changing any output (sum_j dK_j = 0); each row's weights sum to
    one (sum_j dV_j = sum of dO over rows that see a key); the logits depend on
    Q and K only through Q K^T (<Q, dQ> = <K, dK> per KV group);
  * closed forms: one key gives dQ = dK = 0, dV = sum of dO;
  * planted mistakes in the oracle (dropped D term, wrong sign, missing
    scale, dK from P instead of dS, wrong GQA head) each break a pin.
"""


import numpy as np
import pytest
import torch

import oracle
from oracle import backward as oracle_backward

RNG = np.random.default_rng(4321)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def loss(q, k, v, do, scale, causal, window):
    O, _ = oracle.attention_ref(q, k, v, scale, causal, window)
    return float(np.sum(O * do))


def finite_diff(q, k, v, do, scale, causal, window, h=1e-6):
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            up = loss(q, k, v, do, scale, causal, window)
            x[idx] = old - h
            dn = loss(q, k, v, do, scale, causal, window)
            x[idx] = old
            g[idx] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


FD_CASES = [
    # B, Lq, Lk, Hq, Hkv, d, causal, window
    (1, 5, 5, 2, 1, 3, False, (-1, -1)),
    (1, 5, 7, 2, 2, 3, True, (-1, -1)),      # Lk > Lq: bottom-right causal
    (2, 6, 4, 2, 1, 2, True, (-1, -1)),      # Lk < Lq: the first two rows see nothing
    (1, 6, 6, 3, 1, 2, True, (2, 0)),        # sliding window, MQA
    (1, 4, 6, 2, 1, 3, False, (1, 1)),       # two-sided window
]


def fd_check(case, bwd=None):
    B, Lq, Lk, Hq, Hkv, d, causal, window = case
    rng = np.random.default_rng(sum(case[:6]))
    q, k, v = rand(B, Lq, Hq, d, rng=rng), rand(B, Lk, Hkv, d, rng=rng), rand(B, Lk, Hkv, d, rng=rng)
    do = rand(B, Lq, Hq, d, rng=rng)
    scale = 0.7
    got = (bwd or oracle.attention_bwd_ref)(q, k, v, do, scale, causal, window)
    want = finite_diff(q, k, v, do, scale, causal, window)
    return max(float(np.abs(g - w).max()) for g, w in zip(got, want))


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: "-".join(map(str, c[:6])) + f"-c{int(c[6])}-w{c[7][0]}_{c[7][1]}")
def test_matches_finite_differences(case):
    assert fd_check(case) < 1e-7


def torch_grads(q, k, v, do, scale, causal, window):
    """Autograd through a plain masked-softmax attention in float64 (CPU)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kr = kt.repeat_interleave(G, dim=2)
    vr = vt.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", qt, kr) * scale
    i = torch.arange(Lq)[:, None] + (Lk - Lq)
    j = torch.arange(Lk)[None, :]
    vis = torch.ones(Lq, Lk, dtype=torch.bool)
    if causal:
        vis &= j <= i
    if window[0] >= 0:
        vis &= j >= i - window[0]
    if window[1] >= 0:
        vis &= j <= i + window[1]
    p = torch.softmax(s.masked_fill(~vis, float("-inf")), dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, vr)
    (o * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal,window,Hq,Hkv,Lq,Lk", [
    (False, (-1, -1), 4, 2, 37, 37), (True, (-1, -1), 4, 1, 33, 45), (True, (7, 0), 6, 3, 40, 40),
    (False, (5, 9), 2, 2, 30, 26),
])
def test_matches_torch_autograd_fp64(causal, window, Hq, Hkv, Lq, Lk):
    B, d = 2, 16
    q, k, v = rand(B, Lq, Hq, d), rand(B, Lk, Hkv, d), rand(B, Lk, Hkv, d)
    do = rand(B, Lq, Hq, d)
    got = oracle.attention_bwd_ref(q, k, v, do, 0.31, causal, window)
    want = torch_grads(q, k, v, do, 0.31, causal, window)
    for g, w in zip(got, want):
        assert np.abs(g - w).max() < 1e-12 * max(1.0, np.abs(w).max())


def visible_rows(Lq, Lk, causal, window):
    return oracle.key_visibility(Lq, Lk, causal, window[0], window[1]).any(axis=1)


@pytest.mark.parametrize("causal,window,Lq,Lk", [
    (False, (-1, -1), 40, 40), (True, (-1, -1), 50, 31), (True, (10, 0), 40, 52), (False, (3, 3), 20, 20),
])
def test_invariants(causal, window, Lq, Lk):
    B, Hq, Hkv, d = 2, 6, 2, 8
    q, k, v = rand(B, Lq, Hq, d), rand(B, Lk, Hkv, d), rand(B, Lk, Hkv, d)
    do = rand(B, Lq, Hq, d)
    dQ, dK, dV = oracle.attention_bwd_ref(q, k, v, do, 0.45, causal, window)
    G = Hq // Hkv
    seen = visible_rows(Lq, Lk, causal, window)
    for b in range(B):
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            assert np.abs(dK[b, :, g].sum(axis=0)).max() < 1e-10
            want = do[b, seen][:, heads].sum(axis=(0, 1))
            assert np.abs(dV[b, :, g].sum(axis=0) - want).max() < 1e-10
            qdq = np.sum(q[b, :, heads] * dQ[b, :, heads])
            kdk = np.sum(k[b, :, g] * dK[b, :, g])
            assert abs(qdq - kdk) < 1e-10 * max(1.0, abs(qdq))
    assert (dQ[:, ~seen] == 0).all()


def test_single_key_closed_form():
    q, k, v, do = rand(2, 6, 4, 8), rand(2, 1, 2, 8), rand(2, 1, 2, 8), rand(2, 6, 4, 8)
    dQ, dK, dV = oracle.attention_bwd_ref(q, k, v, do, 0.5, False)
    assert np.abs(dQ).max() < 1e-14 and np.abs(dK).max() < 1e-13
    want = do.reshape(2, 6, 2, 2, 8).sum(axis=(1, 3))       # sum over rows and the group's heads
    assert np.abs(dV[:, 0] - want).max() < 1e-12


def test_selected_rows_and_keys_match_the_full_gradient():
    B, Lq, Lk, Hq, Hkv, d = 2, 45, 60, 4, 2, 8
    q, k, v = rand(B, Lq, Hq, d), rand(B, Lk, Hkv, d), rand(B, Lk, Hkv, d)
    do = rand(B, Lq, Hq, d)
    for causal, window in [(True, (-1, -1)), (True, (12, 0)), (False, (-1, -1))]:
        dQ, dK, dV = oracle.attention_bwd_ref(q, k, v, do, 0.3, causal, window, row_block=16)
        rows = [0, 7, 30, 44]
        dq = oracle.attention_bwd_query_rows_ref(q, k, v, do, 1, 3, rows, 0.3, causal, window)
        assert np.abs(dq - dQ[1, rows, 3]).max() < 1e-12
        keys = [0, 14, 15, 59]
        dk, dv = oracle.attention_bwd_key_rows_ref(q, k, v, do, 1, 1, keys, 0.3, causal, window,
                                                   row_block=16)
        assert np.abs(dk - dK[1, keys, 1]).max() < 1e-12
        assert np.abs(dv - dV[1, keys, 1]).max() < 1e-12
        if causal:
            # rows before min(keys) - (Lk - Lq) see none of the keys: skipping them is exact
            late = [40, 41, 59]
            start = min(late) - (Lk - Lq)
            dk2, dv2 = oracle.attention_bwd_key_rows_ref(q, k, v, do, 1, 1, late, 0.3, causal, window,
                                                         row_block=16, row_start=start)
            assert np.abs(dk2 - dK[1, late, 1]).max() < 1e-12
            assert np.abs(dv2 - dV[1, late, 1]).max() < 1e-12


def test_planted_mistakes_are_caught(monkeypatch):
    orig = oracle_backward.attention_bwd_rows

    def no_delta(q_rows, k, v, do_rows, scale, vis):
        o, _, p = oracle.attend_rows(q_rows, k, v, scale, vis)
        ds = p * (do_rows @ v.T)
        return scale * ds @ k, scale * ds.T @ q_rows, p.T @ do_rows

    def wrong_sign(q_rows, k, v, do_rows, scale, vis):
        dq, dk, dv = orig(q_rows, k, v, do_rows, scale, vis)
        return -dq, dk, dv

    def no_scale(q_rows, k, v, do_rows, scale, vis):
        dq, dk, dv = orig(q_rows, k, v, do_rows, scale, vis)
        return dq / scale, dk / scale, dv

    def dk_from_p(q_rows, k, v, do_rows, scale, vis):
        dq, dk, dv = orig(q_rows, k, v, do_rows, scale, vis)
        _, _, p = oracle.attend_rows(q_rows, k, v, scale, vis)
        return dq, scale * (p.T @ q_rows), dv

    cases = [FD_CASES[0], FD_CASES[1], FD_CASES[3]]
    for mut in (no_delta, wrong_sign, no_scale, dk_from_p):
        monkeypatch.setattr(oracle_backward, "attention_bwd_rows", mut)
        assert max(fd_check(c) for c in cases) > 1e-3, mut.__name__
    monkeypatch.setattr(oracle_backward, "attention_bwd_rows", orig)

    # a wrong GQA map (query head h on KV head h % Hkv instead of h // group)
    orig_map = oracle_backward._kv_head
    monkeypatch.setattr(oracle_backward, "_kv_head", lambda h, Hq, Hkv: h % Hkv)
    assert fd_check((1, 5, 5, 4, 2, 3, False, (-1, -1))) > 1e-3
    monkeypatch.setattr(oracle_backward, "_kv_head", orig_map)
    assert max(fd_check(c) for c in cases) < 1e-7


# ------------------------------------------------------------------ varlen
def varlen_loss(q, k, v, do, cq, ck, scale, causal, window):
    O, _ = oracle.attention_varlen_ref(q, k, v, cq, ck, scale, causal, window)
    return float(np.sum(O * do))


def test_varlen_matches_finite_differences():
    # three sequences, one with no rows and one with Lk > Lq
    lq, lk = [3, 0, 2], [2, 3, 4]
    cq = np.concatenate([[0], np.cumsum(lq)]); ck = np.concatenate([[0], np.cumsum(lk)])
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((5, 2, 3)), rng.standard_normal((9, 1, 3)), rng.standard_normal((9, 1, 3))
    do = rng.standard_normal((5, 2, 3))
    got = oracle.attention_varlen_bwd_ref(q, k, v, do, cq, ck, 0.8, True, (2, -1))
    h = 1e-6
    for x, g in zip((q, k, v), got):
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            up = varlen_loss(q, k, v, do, cq, ck, 0.8, True, (2, -1))
            x[idx] = old - h
            dn = varlen_loss(q, k, v, do, cq, ck, 0.8, True, (2, -1))
            x[idx] = old
            assert abs((up - dn) / (2 * h) - g[idx]) < 1e-7


def test_varlen_single_sequence_is_dense_and_sequences_are_isolated():
    q, k, v, do = rand(30, 4, 8), rand(40, 2, 8), rand(40, 2, 8), rand(30, 4, 8)
    got = oracle.attention_varlen_bwd_ref(q, k, v, do, [0, 30], [0, 40], 0.4, True)
    want = oracle.attention_bwd_ref(q[None], k[None], v[None], do[None], 0.4, True)
    for g, w in zip(got, want):
        assert np.abs(g - w[0]).max() < 1e-13
    # changing sequence 1's data leaves sequence 0's gradients unchanged
    cq, ck = [0, 12, 30], [0, 15, 40]
    a = oracle.attention_varlen_bwd_ref(q, k, v, do, cq, ck, 0.4, True)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    q2[12:] += 1.0; k2[15:] -= 2.0; v2[15:] *= 3.0; do2[12:] += 0.5
    b = oracle.attention_varlen_bwd_ref(q2, k2, v2, do2, cq, ck, 0.4, True)
    assert np.array_equal(a[0][:12], b[0][:12]) and np.array_equal(a[1][:15], b[1][:15])
    assert np.array_equal(a[2][:15], b[2][:15])
