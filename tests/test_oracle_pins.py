"""Pins for the CPU oracle: each check ties it to something other than itself.

Kinds of pin used (all CPU, no GPU):
  * library: PyTorch's float64 CPU flash-attention routine, which returns both
    the output and the log-sum-exp, for shapes where its conventions coincide
    with ours (Lq == Lk for causal; any shapes non-causal);
  * closed forms: zero queries make P uniform over the visible keys, so O is the
    mean of the visible V rows and LSE = ln(#visible); causal row 0 sees only
    key 0; constant V rows give that constant; identity V exposes P;
  * invariants named by the pages: GQA broadcast == repeat of KV heads; packed
    varlen == per-sequence calls with no cross-sequence leakage; paged ==
    contiguous; split partials merged == one shot; the streaming online softmax
    == the one-shot softmax;
  * brute force: pure-Python loops with math.fsum on tiny shapes.
A planted-mistake test at the end checks that these pins catch plausible
errors (wrong alignment, dropped scale, wrong GQA map, off-by-one window).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def torch_flash_cpu(q, k, v, scale, causal):
    """PyTorch CPU flash attention in float64; (B, L, H, d) in, O and LSE out."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        qt, kt, vt, 0.0, causal, attn_mask=None, scale=scale)[:2]
    return o.numpy().transpose(0, 2, 1, 3), lse.numpy()


# ------------------------------------------------------------------ library
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (6, 2)])
def test_matches_torch_flash_cpu_fp64(causal, Hq, Hkv):
    B, L, d = 2, 37, 16
    q, k, v = rand(B, L, Hq, d), rand(B, L, Hkv, d), rand(B, L, Hkv, d)
    scale = 0.37
    O, LSE = oracle.attention_ref(q, k, v, scale, causal=causal)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)   # repeat_interleave on heads
    Ot, LSEt = torch_flash_cpu(q, kr, vr, scale, causal)
    assert np.abs(O - Ot).max() < 1e-12
    assert np.abs(LSE - LSEt).max() < 1e-12


def test_matches_torch_noncausal_lq_ne_lk():
    q, k, v = rand(1, 5, 3, 8), rand(1, 23, 3, 8), rand(1, 23, 3, 8)
    O, LSE = oracle.attention_ref(q, k, v, 0.5, causal=False)
    Ot, LSEt = torch_flash_cpu(q, k, v, 0.5, False)
    assert np.abs(O - Ot).max() < 1e-12 and np.abs(LSE - LSEt).max() < 1e-12


def test_default_scale_is_inv_sqrt_d():
    q, k, v = rand(1, 9, 2, 16), rand(1, 9, 2, 16), rand(1, 9, 2, 16)
    O1, _ = oracle.attention_ref(q, k, v, None)
    O2, _ = torch_flash_cpu(q, k, v, 0.25, False)
    assert np.abs(O1 - O2).max() < 1e-12


# ------------------------------------------------------------- closed forms
def test_rows_sum_to_one_and_convex_hull():
    q, k, v = rand(1, 40, 2, 8), rand(1, 40, 2, 8), rand(1, 40, 2, 8)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (True, (5, 0)), (False, (3, 4))]:
        for h in range(2):
            rows = np.arange(40)
            o, lse, p = oracle.attention_rows_ref(q, k, v, 0, h, rows, 0.3, causal, window,
                                                  return_probs=True)
            assert np.abs(p.sum(axis=1) - 1).max() < 1e-12
            vis = oracle.key_visibility(40, 40, causal, *window)
            assert (p[~vis] == 0).all()
            vv = v[0, :, h, :]
            for i in rows:
                lo = vv[vis[i]].min(axis=0) - 1e-12
                hi = vv[vis[i]].max(axis=0) + 1e-12
                assert (o[i] >= lo).all() and (o[i] <= hi).all()


def test_constant_v_returns_constant():
    q, k = rand(2, 17, 4, 8), rand(2, 17, 2, 8)
    c = rand(2, 1, 2, 8)
    v = np.broadcast_to(c, (2, 17, 2, 8)).copy()
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (True, (4, 0))]:
        O, _ = oracle.attention_ref(q, k, v, 0.7, causal, window)
        for h in range(4):
            assert np.abs(O[:, :, h, :] - c[:, :, h // 2, :]).max() < 1e-12


def test_causal_row0_is_v0_and_lse_is_s00():
    q, k, v = rand(1, 12, 1, 8), rand(1, 12, 1, 8), rand(1, 12, 1, 8)
    O, LSE = oracle.attention_ref(q, k, v, 0.4, causal=True)
    assert np.abs(O[0, 0, 0] - v[0, 0, 0]).max() < 1e-14
    assert abs(LSE[0, 0, 0] - 0.4 * float(np.dot(q[0, 0, 0], k[0, 0, 0]))) < 1e-14


def test_zero_q_causal_is_running_mean():
    L = 25
    q = np.zeros((1, L, 1, 8))
    k, v = rand(1, L, 1, 8), rand(1, L, 1, 8)
    O, LSE = oracle.attention_ref(q, k, v, 1.0, causal=True)
    mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, L + 1)[:, None]
    assert np.abs(O[0, :, 0] - mean).max() < 1e-13
    assert np.abs(LSE[0, 0] - np.log(np.arange(1, L + 1))).max() < 1e-13


@pytest.mark.parametrize("W", [0, 1, 3, 10])
def test_zero_q_window_counts_inclusive_bounds(W):
    """window (W, 0): row i sees keys max(0, i-W)..i inclusive, i.e. min(i, W)+1 keys."""
    L = 20
    q = np.zeros((1, L, 1, 4))
    k, v = rand(1, L, 1, 4), rand(1, L, 1, 4)
    O, LSE = oracle.attention_ref(q, k, v, 1.0, causal=True, window=(W, 0))
    for i in range(L):
        lo = max(0, i - W)
        assert abs(LSE[0, 0, i] - math.log(i - lo + 1)) < 1e-13
        assert np.abs(O[0, i, 0] - v[0, lo:i + 1, 0].mean(axis=0)).max() < 1e-13


def test_zero_q_two_sided_window_noncausal():
    L = 15
    q = np.zeros((1, L, 1, 4))
    k, v = rand(1, L, 1, 4), rand(1, L, 1, 4)
    O, LSE = oracle.attention_ref(q, k, v, 1.0, causal=False, window=(2, 3))
    for i in range(L):
        lo, hi = max(0, i - 2), min(L - 1, i + 3)
        assert abs(LSE[0, 0, i] - math.log(hi - lo + 1)) < 1e-13
        assert np.abs(O[0, i, 0] - v[0, lo:hi + 1, 0].mean(axis=0)).max() < 1e-13


def test_window_at_least_length_equals_plain_causal():
    q, k, v = rand(1, 30, 2, 8), rand(1, 30, 2, 8), rand(1, 30, 2, 8)
    a = oracle.attention_ref(q, k, v, 0.3, True, (29, 0))
    b = oracle.attention_ref(q, k, v, 0.3, True, (-1, -1))
    assert np.abs(a[0] - b[0]).max() == 0 and np.abs(a[1] - b[1]).max() == 0


def test_identity_v_exposes_p():
    d = 12
    q, k = rand(1, d, 1, d), rand(1, d, 1, d)
    v = np.eye(d)[None, :, None, :]
    O, _ = oracle.attention_ref(q, k, v, 0.5, causal=True)
    _, _, P = oracle.attention_rows_ref(q, k, v, 0, 0, np.arange(d), 0.5, True, return_probs=True)
    assert np.abs(O[0, :, 0, :] - P).max() < 1e-15
    # and P itself is the softmax of the visible scores of row 2 (keys 0..2)
    s = 0.5 * np.array([np.dot(q[0, 2, 0], k[0, j, 0]) for j in range(3)])
    e = np.exp(s - s.max())
    assert np.abs(P[2, :3] - e / e.sum()).max() < 1e-15 and (P[2, 3:] == 0).all()


def test_lse_bounds():
    q, k, v = rand(1, 33, 1, 8), rand(1, 33, 1, 8), rand(1, 33, 1, 8)
    for causal, window in [(False, (-1, -1)), (True, (7, 0))]:
        _, LSE = oracle.attention_ref(q, k, v, 0.6, causal, window)
        vis = oracle.key_visibility(33, 33, causal, *window)
        s = 0.6 * q[0, :, 0] @ k[0, :, 0].T
        for i in range(33):
            mx = s[i, vis[i]].max()
            assert mx - 1e-12 <= LSE[0, 0, i] <= mx + math.log(vis[i].sum()) + 1e-12


def test_fully_masked_rows_give_zero_and_neg_inf():
    # Lq > Lk with bottom-right causal alignment: the first Lq-Lk rows see nothing.
    q, k, v = rand(1, 6, 1, 4), rand(1, 4, 1, 4), rand(1, 4, 1, 4)
    O, LSE = oracle.attention_ref(q, k, v, 1.0, causal=True)
    assert (O[0, :2] == 0).all() and np.isneginf(LSE[0, 0, :2]).all()
    assert np.isfinite(LSE[0, 0, 2:]).all()


# --------------------------------------------------------------- invariants
def test_gqa_constant_per_kv_head():
    Hq, Hkv = 8, 2
    q, k = rand(1, 10, Hq, 4), rand(1, 10, Hkv, 4)
    c = np.array([3.0, -5.0])
    v = np.zeros((1, 10, Hkv, 4)) + c[None, None, :, None]
    O, _ = oracle.attention_ref(q, k, v, 1.0, causal=True)
    for h in range(Hq):
        assert np.abs(O[0, :, h] - c[h // 4]).max() < 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    Hq, Hkv = 6, 3
    q, k, v = rand(2, 11, Hq, 8), rand(2, 11, Hkv, 8), rand(2, 11, Hkv, 8)
    a = oracle.attention_ref(q, k, v, 0.3, True, (4, 0))
    b = oracle.attention_ref(q, np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2), 0.3, True, (4, 0))
    assert np.abs(a[0] - b[0]).max() == 0 and np.abs(a[1] - b[1]).max() == 0


def test_varlen_equals_per_sequence_and_no_leakage():
    lens = [5, 1, 9, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q, k, v = rand(T, 4, 8), rand(T, 2, 8), rand(T, 2, 8)
    O, LSE = oracle.attention_varlen_ref(q, k, v, cu, cu, 0.4, True, (3, 0))
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        o, lse = oracle.attention_ref(q[None, s:e], k[None, s:e], v[None, s:e], 0.4, True, (3, 0))
        assert np.abs(O[s:e] - o[0]).max() == 0 and np.abs(LSE[:, s:e] - lse[0]).max() == 0
    # perturbing sequence 2's keys/values leaves every other sequence unchanged
    k2, v2 = k.copy(), v.copy()
    k2[cu[2]:cu[3]] += 10.0
    v2[cu[2]:cu[3]] -= 3.0
    O2, LSE2 = oracle.attention_varlen_ref(q, k2, v2, cu, cu, 0.4, True, (3, 0))
    other = np.r_[0:cu[2], cu[3]:T]
    assert np.abs(O2[other] - O[other]).max() == 0


def test_varlen_matches_torch_per_sequence():
    lens = [7, 3, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = rand(cu[-1], 2, 8), rand(cu[-1], 2, 8), rand(cu[-1], 2, 8)
    O, LSE = oracle.attention_varlen_ref(q, k, v, cu, cu, 0.5, True)
    for b in range(3):
        s, e = cu[b], cu[b + 1]
        Ot, LSEt = torch_flash_cpu(q[None, s:e], k[None, s:e], v[None, s:e], 0.5, True)
        assert np.abs(O[s:e] - Ot[0]).max() < 1e-12 and np.abs(LSE[:, s:e] - LSEt[0]).max() < 1e-12


def _paged_from_contiguous(k, v, page_size, rng, pool_extra=3):
    """Scatter per-request contiguous K/V (B, L, Hkv, d) into a random page pool."""
    B, L = k.shape[:2]
    npg = -(-L // page_size)
    pool = B * npg + pool_extra
    perm = rng.permutation(pool)
    kc = np.full((pool, page_size) + k.shape[2:], np.nan)
    vc = np.full((pool, page_size) + k.shape[2:], np.nan)
    table = perm[:B * npg].reshape(B, npg)
    for b in range(B):
        for j in range(L):
            kc[table[b, j // page_size], j % page_size] = k[b, j]
            vc[table[b, j // page_size], j % page_size] = v[b, j]
    return kc, vc, table


def test_paged_decode_equals_last_causal_row():
    rng = np.random.default_rng(7)
    B, L, Hq, Hkv, d, ps = 3, 21, 4, 2, 8, 4
    q_full, k, v = rand(B, L, Hq, d), rand(B, L, Hkv, d), rand(B, L, Hkv, d)
    kc, vc, table = _paged_from_contiguous(k, v, ps, rng)
    O, LSE = oracle.decode_paged_ref(q_full[:, -1:], kc, vc, table, np.full(B, L), ps, 0.3)
    Of, LSEf = oracle.attention_ref(q_full, k, v, 0.3, causal=True)
    assert np.abs(O[:, 0] - Of[:, -1]).max() < 1e-13
    assert np.abs(LSE - LSEf[:, :, -1]).max() < 1e-13
    # also equals the library with the decode row seeing every cached key
    Ot, LSEt = torch_flash_cpu(q_full[:, -1:], np.repeat(k, 2, 2), np.repeat(v, 2, 2), 0.3, False)
    assert np.abs(O - Ot).max() < 1e-12 and np.abs(LSE - LSEt[:, :, 0]).max() < 1e-12


def test_paged_decode_window_and_page_permutation():
    rng = np.random.default_rng(8)
    B, L, Hq, Hkv, d, ps = 2, 19, 2, 1, 4, 3
    q, k, v = rand(B, 1, Hq, d), rand(B, L, Hkv, d), rand(B, L, Hkv, d)
    kc, vc, table = _paged_from_contiguous(k, v, ps, rng)
    lens = np.array([19, 11])
    O, LSE = oracle.decode_paged_ref(q, kc, vc, table, lens, ps, 0.5, window_left=5)
    for b in range(B):
        n = lens[b]
        o, lse = oracle.attention_ref(q[b:b + 1], k[b:b + 1, n - 6:n], v[b:b + 1, n - 6:n], 0.5)
        assert np.abs(O[b] - o[0]).max() < 1e-13 and np.abs(LSE[b] - lse[0, :, 0]).max() < 1e-13
    # re-permute page ids: identical results
    perm = rng.permutation(kc.shape[0])
    inv = np.argsort(perm)
    O2, LSE2 = oracle.decode_paged_ref(q, kc[perm], vc[perm], inv[table], lens, ps, 0.5, 5)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2)


@pytest.mark.parametrize("split", [1, 3, 8, 64])
def test_split_merge_equals_one_shot(split):
    q, k, v = rand(8), rand(37, 8), rand(37, 8)
    lses, outs = oracle.decode_split_partials_ref(q, k, v, 0.4, split)
    lse, o = oracle.merge_partials_ref(lses, outs)
    o1, lse1, _ = oracle.attend_rows(q[None], k, v, 0.4, np.ones((1, 37), bool))
    assert abs(lse - lse1[0]) < 1e-12 and np.abs(o - o1[0]).max() < 1e-12


def test_merge_arbitrary_partition_and_empty():
    rng = np.random.default_rng(3)
    q, k, v = rand(8), rand(50, 8), rand(50, 8)
    cuts = np.sort(rng.choice(np.arange(1, 50), size=6, replace=False))
    bounds = np.concatenate([[0], cuts, [50]])
    lses, outs = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, lse, _ = oracle.attend_rows(q[None], k[a:b], v[a:b], 0.9, np.ones((1, b - a), bool))
        lses.append(lse[0]); outs.append(o[0])
    lse, o = oracle.merge_partials_ref(np.array(lses), np.array(outs))
    o1, lse1, _ = oracle.attend_rows(q[None], k, v, 0.9, np.ones((1, 50), bool))
    assert abs(lse - lse1[0]) < 1e-12 and np.abs(o - o1[0]).max() < 1e-12
    # a partial with no keys (lse = -inf) contributes nothing
    lse2, o2 = oracle.merge_partials_ref(np.array(lses + [-np.inf]), np.array(outs + [np.full(8, 7.0)]))
    assert abs(lse2 - lse) < 1e-15 and np.abs(o2 - o).max() < 1e-15
    lse3, o3 = oracle.merge_partials_ref(np.array([-np.inf]), np.zeros((1, 8)))
    assert np.isneginf(lse3) and (o3 == 0).all()


@pytest.mark.parametrize("block", [1, 4, 16, 100])
def test_online_softmax_equals_one_shot(block):
    q, k, v = rand(8), rand(61, 8), rand(61, 8)
    # rising scores make the running max increase in every block (rescale path)
    k = k + np.linspace(0, 6, 61)[:, None] * q[None] / np.linalg.norm(q)
    o, lse = oracle.online_softmax_ref(q, k, v, 0.5, block)
    o1, lse1, _ = oracle.attend_rows(q[None], k, v, 0.5, np.ones((1, 61), bool))
    assert abs(lse - lse1[0]) < 1e-12 and np.abs(o - o1[0]).max() < 1e-12


# -------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal, wl, wr):
    """Pure-Python loops with math.fsum, one (b, h, i) at a time."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(Lq)] for _ in range(B)]
    LSE = [[[0.0] * Lq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Lq):
                p_i = i + Lk - Lq
                keys = [j for j in range(Lk)
                        if (not causal or j <= p_i) and (wl < 0 or j >= p_i - wl)
                        and (wr < 0 or j <= p_i + wr)]
                if not keys:
                    LSE[b][h][i] = -math.inf
                    continue
                s = {j: scale * math.fsum(q[b, i, h, t] * k[b, j, g, t] for t in range(d)) for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(e.values())
                for t in range(d):
                    O[b][i][h][t] = math.fsum(e[j] * v[b, j, g, t] for j in keys) / l
                LSE[b][h][i] = m + math.log(l)
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (3, 0)),
                                           (False, (2, 1)), (True, (-1, 2))])
@pytest.mark.parametrize("Lq,Lk", [(7, 7), (3, 9), (9, 4)])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_brute_force_dense(causal, window, Lq, Lk, Hq, Hkv):
    q, k, v = rand(2, Lq, Hq, 5), rand(2, Lk, Hkv, 5), rand(2, Lk, Hkv, 5)
    O, LSE = oracle.attention_ref(q, k, v, 0.45, causal, window)
    Ob, LSEb = brute_force(q, k, v, 0.45, causal, *window)
    fin = np.isfinite(LSEb)
    assert np.array_equal(fin, np.isfinite(LSE))
    assert np.abs(LSE[fin] - LSEb[fin]).max() < 1e-12
    assert np.abs(O - Ob).max() < 1e-12


def test_brute_force_varlen_and_paged():
    rng = np.random.default_rng(11)
    lens = [4, 7, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = rand(cu[-1], 4, 3), rand(cu[-1], 2, 3), rand(cu[-1], 2, 3)
    O, LSE = oracle.attention_varlen_ref(q, k, v, cu, cu, 0.8, True, (2, 0))
    for b in range(3):
        s, e = cu[b], cu[b + 1]
        Ob, LSEb = brute_force(q[None, s:e], k[None, s:e], v[None, s:e], 0.8, True, 2, 0)
        assert np.abs(O[s:e] - Ob[0]).max() < 1e-12 and np.abs(LSE[:, s:e] - LSEb[0]).max() < 1e-12
    kk, vv = rand(2, 9, 2, 3), rand(2, 9, 2, 3)
    kc, vc, table = _paged_from_contiguous(kk, vv, 2, rng)
    qd = rand(2, 1, 4, 3)
    O, LSE = oracle.decode_paged_ref(qd, kc, vc, table, np.array([9, 6]), 2, 0.8)
    for b, n in enumerate([9, 6]):
        Ob, LSEb = brute_force(qd[b:b + 1], kk[b:b + 1, :n], vv[b:b + 1, :n], 0.8, True, -1, -1)
        assert np.abs(O[b] - Ob[0]).max() < 1e-12 and np.abs(LSE[b] - LSEb[0, :, 0]).max() < 1e-12


# ------------------------------------------- KV cache: append + chunked prefill
def brute_force_kvcache(q, kc, vc, table, lens, ps, k_new, v_new, scale, causal, wl, wr):
    """Pure-Python loops: new rows written slot by slot at position lens[b] + i,
    then every (b, h, i) attends over the request's positions through the page
    table, query row i sitting at position i + n - Lq."""
    kc, vc = kc.copy(), vc.copy()
    B, Lq, Hq, d = q.shape
    Hkv = kc.shape[2]
    G = Hq // Hkv
    if k_new is not None:
        for b in range(B):
            for i in range(Lq):
                pos = int(lens[b]) + i
                pg, sl = int(table[b][pos // ps]), pos % ps
                for g in range(Hkv):
                    for t in range(d):
                        kc[pg, sl, g, t] = k_new[b, i, g, t]
                        vc[pg, sl, g, t] = v_new[b, i, g, t]
    O = np.zeros((B, Lq, Hq, d))
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        n = int(lens[b]) + (Lq if k_new is not None else 0)
        for h in range(Hq):
            g = h // G
            for i in range(Lq):
                p_i = i + n - Lq
                keys = [j for j in range(n)
                        if (not causal or j <= p_i) and (wl < 0 or j >= p_i - wl)
                        and (wr < 0 or j <= p_i + wr)]
                if not keys:
                    LSE[b, h, i] = -math.inf
                    continue
                row = {j: (int(table[b][j // ps]), j % ps) for j in keys}
                s = {j: scale * math.fsum(q[b, i, h, t] * kc[row[j][0], row[j][1], g, t] for t in range(d))
                     for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(e.values())
                for t in range(d):
                    O[b, i, h, t] = math.fsum(e[j] * vc[row[j][0], row[j][1], g, t] for j in keys) / l
                LSE[b, h, i] = m + math.log(l)
    return O, LSE, kc, vc


def _kvcache_case(seed, B=2, Lq=3, Hq=4, Hkv=2, d=3, ps=2, lens=(5, 2), npages=6):
    rng = np.random.default_rng(seed)
    pool = B * npages + 2
    kc = rng.standard_normal((pool, ps, Hkv, d))
    vc = rng.standard_normal((pool, ps, Hkv, d))
    table = rng.permutation(pool)[:B * npages].reshape(B, npages)
    q = rng.standard_normal((B, Lq, Hq, d))
    kn = rng.standard_normal((B, Lq, Hkv, d))
    vn = rng.standard_normal((B, Lq, Hkv, d))
    return q, kc, vc, table, np.array(lens), ps, kn, vn


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (2, 0)), (False, (-1, -1)),
                                           (False, (1, 1))])
def test_brute_force_kvcache(append, causal, window):
    q, kc, vc, table, lens, ps, kn, vn = _kvcache_case(21)
    if not append:
        kn = vn = None
        lens = np.array([7, 4])
    O, LSE, kc2, vc2 = oracle.attention_kvcache_ref(q, kc, vc, table, lens, ps, kn, vn, 0.6, causal, window)
    Ob, LSEb, kcb, vcb = brute_force_kvcache(q, kc, vc, table, lens, ps, kn, vn, 0.6, causal, *window)
    fin = np.isfinite(LSEb)
    assert np.array_equal(fin, np.isfinite(LSE))
    assert np.abs(LSE[fin] - LSEb[fin]).max() < 1e-12
    assert np.abs(O - Ob).max() < 1e-12
    assert np.array_equal(kc2, kcb) and np.array_equal(vc2, vcb)


def test_kvcache_equals_contiguous_attention():
    rng = np.random.default_rng(22)
    B, L0, Lq, Hq, Hkv, d, ps = 2, 13, 6, 4, 2, 8, 4
    k_all, v_all = rand(B, L0 + Lq, Hkv, d), rand(B, L0 + Lq, Hkv, d)
    q = rand(B, Lq, Hq, d)
    # cache holds the first L0 tokens; pages for the appended ones exist but hold NaN
    kc, vc, table = _paged_from_contiguous(k_all[:, :L0], v_all[:, :L0], ps, rng, pool_extra=12)
    npg = -(-(L0 + Lq) // ps)
    free = [p for p in range(kc.shape[0]) if p not in set(table.ravel())]
    table = np.concatenate([table, np.array(free[:B * (npg - table.shape[1])]).reshape(B, -1)], 1)
    lens = np.full(B, L0)
    for causal, window in [(True, (-1, -1)), (True, (5, 0)), (False, (-1, -1))]:
        O, LSE, kc2, vc2 = oracle.attention_kvcache_ref(q, kc, vc, table, lens, ps, k_all[:, L0:],
                                                        v_all[:, L0:], 0.35, causal, window)
        Of, LSEf = oracle.attention_ref(q, k_all, v_all, 0.35, causal, window)
        assert np.abs(O - Of).max() < 1e-13 and np.abs(LSE - LSEf).max() < 1e-13
    # the appended rows are where positions L0 .. L0+Lq-1 say
    for b in range(B):
        assert np.array_equal(oracle.gather_paged(kc2, table[b], L0 + Lq, ps), k_all[b])
    # without new rows: the queries sit at the last Lq cached positions
    O, LSE, kc3, _ = oracle.attention_kvcache_ref(q, kc2, vc2, table, np.full(B, L0 + Lq), ps,
                                                  None, None, 0.35, True)
    Of, LSEf = oracle.attention_ref(q, k_all, v_all, 0.35, True)
    assert kc3 is kc2
    assert np.abs(O - Of).max() < 1e-13 and np.abs(LSE - LSEf).max() < 1e-13


def test_kvcache_single_query_row_equals_decode():
    rng = np.random.default_rng(23)
    B, L, Hq, Hkv, d, ps = 3, 17, 4, 1, 8, 4
    k, v = rand(B, L, Hkv, d), rand(B, L, Hkv, d)
    kc, vc, table = _paged_from_contiguous(k, v, ps, rng)
    q = rand(B, 1, Hq, d)
    lens = np.array([17, 9, 1])
    O, LSE, _, _ = oracle.attention_kvcache_ref(q, kc, vc, table, lens, ps, None, None, 0.5, True)
    Od, LSEd = oracle.decode_paged_ref(q, kc, vc, table, lens, ps, 0.5)
    assert np.abs(O - Od).max() < 1e-13 and np.abs(LSE[:, :, 0] - LSEd).max() < 1e-13


def test_append_touches_only_the_new_slots():
    q, kc, vc, table, lens, ps, kn, vn = _kvcache_case(24)
    kc2, vc2 = oracle.append_paged_ref(kc, vc, kn, vn, table, lens, ps)
    changed = ~np.all(kc2 == kc, axis=(2, 3))
    expect = np.zeros_like(changed)
    for b in range(len(lens)):
        for i in range(kn.shape[1]):
            pos = lens[b] + i
            expect[table[b][pos // ps], pos % ps] = True
    assert np.array_equal(changed, expect)
    assert np.array_equal(~np.all(vc2 == vc, axis=(2, 3)), expect)
    assert not np.shares_memory(kc2, kc)


def test_kvcache_planted_mistakes_are_caught(monkeypatch):
    q, kc, vc, table, lens, ps, kn, vn = _kvcache_case(25)
    Ob, LSEb, _, _ = brute_force_kvcache(q, kc, vc, table, lens, ps, kn, vn, 0.6, True, -1, -1)
    orig_append, orig_gather = oracle_attention.append_paged_ref, oracle_attention.gather_paged

    def append_off_by_one(k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, page_size):
        return orig_append(k_cache, v_cache, k_new, v_new, block_table, np.asarray(cache_seqlens) - 1, page_size)

    def gather_shifted(cache, block_table_row, length, page_size):
        j = np.arange(length, dtype=np.int64) + 1
        return cache[np.asarray(block_table_row, dtype=np.int64)[j // page_size], j % page_size]

    for name, mut in [("append_paged_ref", append_off_by_one), ("gather_paged", gather_shifted)]:
        monkeypatch.setattr(oracle_attention, name, mut)
        O, LSE, _, _ = oracle_attention.attention_kvcache_ref(q, kc, vc, table, lens, ps, kn, vn, 0.6, True)
        assert np.abs(O - Ob).max() > 1e-3, name
        monkeypatch.setattr(oracle_attention, "append_paged_ref", orig_append)
        monkeypatch.setattr(oracle_attention, "gather_paged", orig_gather)


# ---------------------------------------------------- softcap and ALiBi slopes
def test_softcap_large_cap_is_plain_attention():
    q, k, v = rand(2, 9, 4, 8), rand(2, 11, 2, 8), rand(2, 11, 2, 8)
    O, LSE = oracle.attention_ref(q, k, v, 0.4, True)
    Oc, LSEc = oracle.attention_ref(q, k, v, 0.4, True, softcap=1e9)
    assert np.abs(O - Oc).max() < 1e-9 and np.abs(LSE - LSEc).max() < 1e-9


def test_softcap_saturation_gives_mean_and_cap_plus_log_count():
    # every logit ~ +1e4: tanh saturates, each visible key scores exactly cap
    d, L = 8, 12
    u = np.ones(d) / math.sqrt(d)
    k = (40.0 * u + 1e-3 * rand(L, d))[None, :, None, :]
    q = (1e4 * u)[None, None, None, :].repeat(L, 1)
    v = rand(1, L, 1, d)
    O, LSE = oracle.attention_ref(q, k, v, 1.0, True, softcap=3.0)
    for i in range(L):
        assert np.abs(O[0, i, 0] - v[0, :i + 1, 0].mean(0)).max() < 1e-12
        assert abs(LSE[0, 0, i] - (3.0 + math.log(i + 1))) < 1e-12


def test_alibi_zero_slopes_is_plain_attention():
    q, k, v = rand(2, 7, 4, 8), rand(2, 10, 2, 8), rand(2, 10, 2, 8)
    O, LSE = oracle.attention_ref(q, k, v, 0.4, False, (3, 2))
    Oa, LSEa = oracle.attention_ref(q, k, v, 0.4, False, (3, 2), alibi_slopes=np.zeros(4))
    assert np.array_equal(O, Oa) and np.array_equal(LSE, LSEa)


@pytest.mark.parametrize("slope", [0.05, 0.5, 2.0])
def test_alibi_zero_q_closed_form(slope):
    # Q = 0: logits are -slope * (pos_i - j) over the causal keys j <= pos_i, a
    # geometric series: LSE = ln sum_{t=0}^{pos} e^{-slope t}; identity V exposes P
    Lq, Lk = 5, 9
    q = np.zeros((1, Lq, 2, Lk))
    k = rand(1, Lk, 1, Lk)
    v = np.eye(Lk)[None, :, None, :]
    O, LSE = oracle.attention_ref(q, k, v, 0.7, True, alibi_slopes=np.array([slope, 2 * slope]))
    for h, sl in enumerate([slope, 2 * slope]):
        for i in range(Lq):
            pos = i + Lk - Lq
            z = (1 - math.exp(-sl * (pos + 1))) / (1 - math.exp(-sl))
            assert abs(LSE[0, h, i] - math.log(z)) < 1e-12
            want = np.array([math.exp(-sl * (pos - j)) / z if j <= pos else 0.0 for j in range(Lk)])
            assert np.abs(O[0, i, h] - want).max() < 1e-13


def brute_force_mod(q, k, v, scale, causal, wl, wr, softcap, slopes):
    """brute_force with the score modifiers written out per score."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Lq, Hq, d))
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            sl = slopes[h] if slopes.ndim == 1 else slopes[b, h]
            for i in range(Lq):
                p_i = i + Lk - Lq
                keys = [j for j in range(Lk)
                        if (not causal or j <= p_i) and (wl < 0 or j >= p_i - wl)
                        and (wr < 0 or j <= p_i + wr)]
                if not keys:
                    LSE[b, h, i] = -math.inf
                    continue
                s = {}
                for j in keys:
                    x = scale * math.fsum(q[b, i, h, t] * k[b, j, g, t] for t in range(d))
                    if softcap > 0:
                        x = softcap * math.tanh(x / softcap)
                    s[j] = x - sl * abs(p_i - j)
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(e.values())
                for t in range(d):
                    O[b, i, h, t] = math.fsum(e[j] * v[b, j, g, t] for j in keys) / l
                LSE[b, h, i] = m + math.log(l)
    return O, LSE


@pytest.mark.parametrize("softcap", [0.0, 0.8])
@pytest.mark.parametrize("per_batch", [False, True])
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (2, 1))])
def test_brute_force_softcap_alibi(softcap, per_batch, causal, window):
    rng = np.random.default_rng(31)
    q, k, v = rand(2, 5, 4, 3), rand(2, 8, 2, 3), rand(2, 8, 2, 3)
    slopes = rng.uniform(0.0, 0.6, (2, 4) if per_batch else 4)
    O, LSE = oracle.attention_ref(q, k, v, 0.9, causal, window, softcap=softcap, alibi_slopes=slopes)
    Ob, LSEb = brute_force_mod(q, k, v, 0.9, causal, *window, softcap, slopes)
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(LSE - LSEb).max() < 1e-12


def test_modifiers_varlen_and_kvcache_match_dense():
    rng = np.random.default_rng(32)
    lens = [4, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = rand(cu[-1], 4, 3), rand(cu[-1], 2, 3), rand(cu[-1], 2, 3)
    slopes = rng.uniform(0.1, 0.5, (3, 4))
    O, LSE = oracle.attention_varlen_ref(q, k, v, cu, cu, 0.8, True, softcap=1.5, alibi_slopes=slopes)
    for b in range(3):
        s, e = cu[b], cu[b + 1]
        Ob, LSEb = brute_force_mod(q[None, s:e], k[None, s:e], v[None, s:e], 0.8, True, -1, -1,
                                   1.5, slopes[b])
        assert np.abs(O[s:e] - Ob[0]).max() < 1e-12 and np.abs(LSE[:, s:e] - LSEb[0]).max() < 1e-12
    qc, kc, vc, table, lens2, ps, kn, vn = _kvcache_case(33)
    Okv, LSEkv, kc2, vc2 = oracle.attention_kvcache_ref(qc, kc, vc, table, lens2, ps, kn, vn, 0.6, True,
                                                        softcap=2.0, alibi_slopes=slopes[:2])
    for b in range(2):
        n = lens2[b] + qc.shape[1]
        kk = oracle.gather_paged(kc2, table[b], n, ps)[None]
        vv = oracle.gather_paged(vc2, table[b], n, ps)[None]
        Ob, LSEb = brute_force_mod(qc[b:b + 1], kk, vv, 0.6, True, -1, -1, 2.0, slopes[b])
        assert np.abs(Okv[b] - Ob[0]).max() < 1e-12 and np.abs(LSEkv[b] - LSEb[0]).max() < 1e-12


@pytest.mark.parametrize("window_left", [-1, 3])
def test_modifiers_decode_match_brute_force(window_left):
    # one query row per request at position len - 1 over a paged cache
    rng = np.random.default_rng(34)
    ps, lens = 4, [7, 1, 10]
    perm = rng.permutation(8)
    table = np.zeros((3, 3), dtype=np.int32)
    table[0, :2], table[1, :1], table[2, :3] = perm[0:2], perm[2:3], perm[3:6]
    kc, vc = rand(8, ps, 2, 3), rand(8, ps, 2, 3)
    q = rand(3, 1, 4, 3)
    slopes = rng.uniform(0.1, 0.6, (3, 4))
    O, LSE = oracle.decode_paged_ref(q, kc, vc, table, lens, ps, 0.9, window_left, softcap=0.7,
                                     alibi_slopes=slopes)
    for b, n in enumerate(lens):
        kk = oracle.gather_paged(kc, table[b], n, ps)[None]
        vv = oracle.gather_paged(vc, table[b], n, ps)[None]
        Ob, LSEb = brute_force_mod(q[b:b + 1], kk, vv, 0.9, True, window_left, -1, 0.7, slopes[b])
        assert np.abs(O[b] - Ob[0]).max() < 1e-12 and np.abs(LSE[b] - LSEb[0, :, 0]).max() < 1e-12


def test_modifier_planted_mistakes_are_caught(monkeypatch):
    orig_bias, orig_attend = oracle_attention.alibi_bias, oracle_attention.attend_rows

    def bias_wrong_sign(rows, Lq, Lk, slope):
        return -orig_bias(rows, Lq, Lk, slope)

    def bias_top_left(rows, Lq, Lk, slope):
        return orig_bias(rows, Lk, Lk, slope)

    def cap_before_scale(q_rows, k, v, scale, vis, softcap=0.0, bias=None):
        if softcap <= 0:
            return orig_attend(q_rows, k, v, scale, vis, softcap, bias)
        s = softcap * np.tanh((np.asarray(q_rows, float) @ np.asarray(k, float).T) / softcap)
        qq = np.asarray(q_rows, float) * 0   # recompute: scale applied after the cap
        o, lse, p = orig_attend(qq, k, v, 1.0, vis, 0.0, scale * s + (0 if bias is None else bias))
        return o, lse, p

    checks = [
        ("alibi_bias", bias_wrong_sign, lambda: test_alibi_zero_q_closed_form(0.5)),
        ("alibi_bias", bias_top_left, lambda: test_alibi_zero_q_closed_form(0.5)),
        ("attend_rows", cap_before_scale, lambda: test_brute_force_softcap_alibi(0.8, False, True, (-1, -1))),
    ]
    for name, mut, pin in checks:
        monkeypatch.setattr(oracle_attention, name, mut)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.setattr(oracle_attention, "alibi_bias", orig_bias)
        monkeypatch.setattr(oracle_attention, "attend_rows", orig_attend)


# ---------------------------------------------------------- planted mistakes
def _pin_suite(attn):
    """A few pins rerun against a (possibly mutated) attention function; returns
    the list of pins that failed."""
    failed = []
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((1, 12, 4, 8)), r.standard_normal((1, 12, 2, 8)), r.standard_normal((1, 12, 2, 8))
    O, LSE = attn(q, k, v, 0.3, True, (-1, -1))
    Ot, LSEt = torch_flash_cpu(q, np.repeat(k, 2, 2), np.repeat(v, 2, 2), 0.3, True)
    if not (np.abs(O - Ot).max() < 1e-12 and np.abs(LSE - LSEt).max() < 1e-12):
        failed.append("torch")
    z = np.zeros((1, 10, 1, 4))
    kz, vz = r.standard_normal((1, 10, 1, 4)), r.standard_normal((1, 10, 1, 4))
    _, LSEz = attn(z, kz, vz, 1.0, True, (3, 0))
    if np.abs(LSEz[0, 0] - np.log(np.minimum(np.arange(10), 3) + 1)).max() > 1e-12:
        failed.append("window-count")
    qd, kd, vd = r.standard_normal((1, 1, 2, 4)), r.standard_normal((1, 6, 2, 4)), r.standard_normal((1, 6, 2, 4))
    Od, _ = attn(qd, kd, vd, 0.5, True, (-1, -1))       # decode row must see all 6 keys
    Odt, _ = torch_flash_cpu(qd, kd, vd, 0.5, False)
    if np.abs(Od - Odt).max() > 1e-12:
        failed.append("decode-alignment")
    return failed


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pin_suite(lambda *a: oracle.attention_ref(*a)) == []
    orig_vis = oracle_attention.key_visibility
    orig_attend = oracle_attention.attend_rows
    orig_head = oracle_attention._kv_head

    def top_left(Lq, Lk, causal, wl=-1, wr=-1, rows=None):
        return orig_vis(Lk, Lk, causal, wl, wr, rows=rows)        # drops the Lk-Lq shift

    def off_by_one(Lq, Lk, causal, wl=-1, wr=-1, rows=None):
        return orig_vis(Lq, Lk, causal, wl + 1 if wl >= 0 else wl, wr, rows=rows)

    def no_scale(q_rows, k, v, scale, vis, softcap=0.0, bias=None):
        return orig_attend(q_rows, k, v, 1.0, vis, softcap, bias)

    def modulo_heads(h, Hq, Hkv):
        return h % Hkv

    def v_transposed(q_rows, k, v, scale, vis, softcap=0.0, bias=None):
        o, lse, p = orig_attend(q_rows, k, v, scale, vis, softcap, bias)
        return (p @ np.asarray(v)[::-1], lse, p)                  # wrong V rows

    for name, mut in [("key_visibility", top_left), ("key_visibility", off_by_one),
                      ("attend_rows", no_scale), ("_kv_head", modulo_heads),
                      ("attend_rows", v_transposed)]:
        monkeypatch.setattr(oracle_attention, name, mut)
        assert _pin_suite(lambda *a: oracle_attention.attention_ref(*a)) != [], (name, mut.__name__)
        monkeypatch.setattr(oracle_attention, "key_visibility", orig_vis)
        monkeypatch.setattr(oracle_attention, "attend_rows", orig_attend)
        monkeypatch.setattr(oracle_attention, "_kv_head", orig_head)


def test_uint16_inputs_are_bf16_bit_patterns():
    x = np.array([1.0, -2.5, 3.140625, 0.0, 65280.0], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)            # exact bf16 values
    q = bits.reshape(1, 1, 1, 5)
    k = np.ones((1, 1, 1, 5))
    v = bits.reshape(1, 1, 1, 5)
    O, _ = oracle.attention_ref(q, k, v, 1.0)
    assert np.array_equal(O[0, 0, 0], x.astype(np.float64))


# ------------------------------------------------ sampled-row checker pins
# attention_rows_ref checks every full-size prefill output on the GPU, so it is
# pinned on its own: against the per-score brute force (which shares none of
# its code) at b > 0, GQA heads, Lq != Lk, windows and both score modifiers,
# and against attention_ref's rows on shapes with several row blocks.
ROWS_CASES = [
    # B, Lq, Lk, Hq, Hkv, causal, window, softcap, slopes shape
    (3, 9, 9, 4, 2, True, (-1, -1), 0.0, None),
    (2, 5, 11, 6, 2, True, (3, 0), 0.0, None),        # Lq < Lk, window, G = 3
    (2, 10, 6, 4, 1, True, (-1, -1), 0.0, None),      # Lq > Lk: leading rows see no key
    (3, 8, 8, 4, 4, False, (2, 1), 0.0, None),
    (2, 7, 9, 4, 2, True, (-1, 2), 0.7, "h"),
    (3, 6, 6, 6, 3, False, (-1, -1), 0.0, "bh"),
    (2, 9, 12, 4, 2, True, (4, 0), 1.3, "bh"),
]


@pytest.mark.parametrize("case", ROWS_CASES)
def test_rows_checker_matches_brute_force(case):
    B, Lq, Lk, Hq, Hkv, causal, window, softcap, sh = case
    rng = np.random.default_rng(400 + Lq * Lk + Hq)
    d = 4
    q, k, v = rng.standard_normal((B, Lq, Hq, d)), rng.standard_normal((B, Lk, Hkv, d)), \
        rng.standard_normal((B, Lk, Hkv, d))
    slopes = None if sh is None else rng.uniform(0.05, 0.7, Hq if sh == "h" else (B, Hq))
    Ob, LSEb = brute_force_mod(q, k, v, 0.6, causal, *window, softcap,
                               np.zeros(Hq) if slopes is None else slopes)
    for b in range(B):
        for h in range(Hq):
            rows = rng.permutation(Lq)[:max(1, Lq // 2 + 1)]
            O, LSE = oracle.attention_rows_ref(q, k, v, b, h, rows, 0.6, causal, window,
                                               softcap=softcap, alibi_slopes=slopes)
            want = LSEb[b, h, rows]
            fin = np.isfinite(want)
            assert np.array_equal(np.isfinite(LSE), fin), (b, h, rows)
            assert np.abs(LSE[fin] - want[fin]).max(initial=0.0) < 1e-12
            assert np.abs(O - Ob[b, rows, h]).max() < 1e-12


@pytest.mark.parametrize("causal,window,softcap,sh", [(True, (-1, -1), 0.0, None),
                                                       (True, (300, 0), 0.0, None),
                                                       (False, (40, 90), 2.0, "bh"),
                                                       (True, (-1, -1), 0.0, "h")])
def test_rows_checker_matches_full_oracle_across_row_blocks(causal, window, softcap, sh):
    """Rows on both sides of attention_ref's 1024-row block boundary, at b > 0
    and on every query head of a GQA group."""
    rng = np.random.default_rng(77)
    B, Lq, Lk, Hq, Hkv, d = 2, 1100, 1300, 4, 2, 8
    q, k, v = rng.standard_normal((B, Lq, Hq, d)), rng.standard_normal((B, Lk, Hkv, d)), \
        rng.standard_normal((B, Lk, Hkv, d))
    slopes = None if sh is None else rng.uniform(0.0, 0.05, Hq if sh == "h" else (B, Hq))
    O, LSE = oracle.attention_ref(q, k, v, 0.3, causal, window, softcap=softcap,
                                  alibi_slopes=slopes)
    rows = np.array([0, 1, 511, 1022, 1023, 1024, 1025, Lq - 1])
    for b in range(B):
        for h in range(Hq):
            Or, LSEr = oracle.attention_rows_ref(q, k, v, b, h, rows, 0.3, causal, window,
                                                 softcap=softcap, alibi_slopes=slopes)
            assert np.abs(Or - O[b, rows, h]).max() < 1e-12
            assert np.abs(LSEr - LSE[b, h, rows]).max() < 1e-12


def test_rows_checker_planted_mistakes_are_caught(monkeypatch):
    """Mistakes a sampled-row checker could make -- reading batch 0, the wrong KV
    head, rows counted from the top instead of bottom-right -- fail the pins."""
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((2, 5, 4, 3)), rng.standard_normal((2, 8, 2, 3)), \
        rng.standard_normal((2, 8, 2, 3))
    Ob, LSEb = brute_force_mod(q, k, v, 0.8, True, -1, -1, 0.0, np.zeros(4))

    def agrees(fn):
        rows = np.arange(5)
        for b in range(2):
            for h in range(4):
                O, _ = fn(q, k, v, b, h, rows, 0.8, True)
                if np.abs(O - Ob[b, rows, h]).max() > 1e-12:
                    return False
        return True

    assert agrees(oracle.attention_rows_ref)
    orig = oracle_attention.attention_rows_ref
    assert not agrees(lambda q_, k_, v_, b, h, rows, *a: orig(q_, k_, v_, 0, h, rows, *a))
    assert not agrees(lambda q_, k_, v_, b, h, rows, *a: orig(q_, k_, v_, b, h % 2 * 2, rows, *a))
    orig_vis = oracle_attention.key_visibility
    monkeypatch.setattr(oracle_attention, "key_visibility",
                        lambda Lq, Lk, c, wl=-1, wr=-1, rows=None: orig_vis(Lk, Lk, c, wl, wr, rows=rows))
    assert not agrees(oracle_attention.attention_rows_ref)
