"""Gradients of dense attention in float64 on the CPU (test infrastructure only).

The pages say what the backward pass of fused attention does -- it keeps no
score matrix from the forward pass and recomputes the blocks it needs from the
saved row statistics ("FlashAttention" concept page, sec. on recomputation;
"FIA / FlashAttention" explainer, sec. 1) -- but print no formula for the
gradients.  The values are fixed by the forward definition alone: this module
writes out the derivative of

    O = P V,  P = softmax(scale * Q K^T + mask) row-wise

with respect to Q, K and V for an upstream gradient dO, by the chain rule:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij  (= dO_i . O_i)
    dS = P * (dP - D)          (gradient of the logits; the softmax Jacobian)
    dQ = scale * dS K,   dK = scale * dS^T Q.

With grouped KV heads (GQA), query head h reads KV head h // (Hq // Hkv), so
dK and dV of a KV head sum the contributions of its query heads.  A query row
with no visible key has O = 0 whatever Q, K, V are, so its contributions are
zero.  Nothing is blocked or recomputed here: P is formed whole per (batch,
head) from the forward definition (``attend_rows``); row blocks only bound
memory.
"""

import math

import numpy as np

from .attention import _f64, _kv_head, attend_rows, key_visibility


def attention_bwd_rows(q_rows, k, v, do_rows, scale, vis):
    """Gradient contributions of a block of query rows of one head.

    q_rows, do_rows: (n, d); k, v: (Lk, d); vis: (n, Lk) bool.
    Returns dq_rows (n, d), dk (Lk, d), dv (Lk, dv) -- the latter two are this
    block's share, to be summed over blocks and over the heads of a group.
    """
    o, _, p = attend_rows(q_rows, k, v, scale, vis)     # p = 0 where masked or for empty rows
    dv = p.T @ do_rows
    dp = do_rows @ v.T
    D = np.sum(do_rows * o, axis=1, keepdims=True)
    ds = p * (dp - D)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q_rows)
    return dq, dk, dv


def attention_bwd_ref(q, k, v, dout, softmax_scale=None, causal=False, window=(-1, -1),
                      row_block=1024):
    """dQ, dK, dV (float64) of dense attention over (B, L, H, d) tensors for the
    upstream gradient dout (B, Lq, Hq, d).  Masks as in ``attention_ref``."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Lk, Hkv, d) or v.shape[:3] != (B, Lk, Hkv) or dout.shape != q.shape:
        raise ValueError("q/k/v/dout shapes disagree")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            for r0 in range(0, Lq, row_block):
                rows = np.arange(r0, min(Lq, r0 + row_block))
                vis = key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
                dq, dk, dv = attention_bwd_rows(q[b, rows, h], k[b, :, g], v[b, :, g],
                                                dout[b, rows, h], scale, vis)
                dQ[b, rows, h] = dq
                dK[b, :, g] += dk
                dV[b, :, g] += dv
    return dQ, dK, dV


def attention_bwd_query_rows_ref(q, k, v, dout, b, h, rows, softmax_scale=None, causal=False,
                                 window=(-1, -1)):
    """dQ of selected query rows of one (batch, query head): (n, d)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    vis = key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
    dq, _, _ = attention_bwd_rows(_f64(q[b, rows, h]), _f64(k[b, :, g]), _f64(v[b, :, g]),
                                  _f64(dout[b, rows, h]), scale, vis)
    return dq


def attention_bwd_key_rows_ref(q, k, v, dout, b, g, keys, softmax_scale=None, causal=False,
                               window=(-1, -1), row_block=1024, row_start=0):
    """dK and dV of selected key rows of one (batch, KV head g): (n, d) each.

    Every query row of every query head of the group contributes, so all rows
    are visited (in blocks); each block's P is formed over all keys (the row
    normalisation needs them) and only the selected key columns are kept.
    Rows before ``row_start`` are skipped: pass it only when those rows see
    none of the selected keys (e.g. causal, row_start <= min(keys) - (Lk - Lq)),
    so that their contribution is zero.
    """
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    keys = np.asarray(keys, dtype=np.int64)
    kk, vv = _f64(k[b, :, g]), _f64(v[b, :, g])
    dk = np.zeros((keys.size, d))
    dv = np.zeros((keys.size, v.shape[3]))
    group = Hq // Hkv
    for h in range(g * group, (g + 1) * group):
        for r0 in range(row_start, Lq, row_block):
            rows = np.arange(r0, min(Lq, r0 + row_block))
            vis = key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
            qr, dr = _f64(q[b, rows, h]), _f64(dout[b, rows, h])
            o, _, p = attend_rows(qr, kk, vv, scale, vis)
            dp = dr @ vv[keys].T
            D = np.sum(dr * o, axis=1, keepdims=True)
            ds = p[:, keys] * (dp - D)
            dk += scale * (ds.T @ qr)
            dv += p[:, keys].T @ dr
    return dk, dv


def attention_varlen_bwd_ref(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, softmax_scale=None,
                             causal=False, window=(-1, -1), row_block=1024):
    """dQ, dK, dV (float64) of packed varlen attention: q, dout (total_q, Hq, d),
    k, v (total_k, Hkv, d).  Sequences never attend across each other, so the
    gradient of sequence b is the dense gradient of its own slices."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cq) - 1):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        if cq[b + 1] == cq[b] or ck[b + 1] == ck[b]:
            continue    # no rows or no keys: every gradient of the sequence is 0
        g = attention_bwd_ref(q[None, qs], k[None, ks], v[None, ks], dout[None, qs], scale,
                              causal, window, row_block)
        dQ[qs], dK[ks], dV[ks] = g[0][0], g[1][0], g[2][0]
    return dQ, dK, dV
