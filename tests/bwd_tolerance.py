"""Elementwise error bounds for the backward kernels (test helper, not collected).

The bound follows the arithmetic of the HIP path, to first order in the bf16
unit roundoff u = 2^-8 (round to nearest even, 8 significant bits):

  * P is recomputed in fp32 from bf16 Q, K and the forward's fp32 LSE
    (relative error ~1e-4 at most, from the LSE) and rounded to bf16 for
    dV = P^T dO:                           |dP_err| <= (u + 1e-4) P
  * delta_i = dO_i . O_i uses the forward kernel's bf16 output O, whose own
    error (its bf16 P, then the output rounding) is at most
    2u sum_j P_ij |V_jd|:                  |delta_err| <= 2u sum_d |dO_id| (P |V|)_id
  * dS = P (dP - delta) is rounded to bf16: |dS_err| <= (u + 1e-4) |dS| + P |delta_err|
  * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO accumulate in fp32 and are
    rounded to bf16 on output (u |g|).

So |dV_j err| <= (u + 1e-4) sum_i P_ij |dO_i| + u |dV_j|,
   |dQ_i err| <= scale sum_j |dS_err_ij| |K_j| + u |dQ_i|,
   |dK_j err| <= scale sum_i |dS_err_ij| |Q_i| + u |dK_j|,
summed over the query heads of a KV group for dK and dV.  The tests allow
twice this bound plus 1e-5 (fp32 accumulation order, outputs that are 0).
The quantities P, O, dP and delta come from the float64 oracle.
"""

import math

import numpy as np

import oracle

U = 2.0 ** -8
LSE_REL = 1e-4


def _f64(x):
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _block_terms(q_rows, k, v, do_rows, scale, vis):
    """P and the bound on dS for one block of query rows of one head."""
    o, _, p = oracle.attend_rows(q_rows, k, v, scale, vis)
    dp = do_rows @ v.T
    D = np.sum(do_rows * o, axis=1, keepdims=True)
    ds = p * (dp - D)
    ddelta = 2 * U * np.sum(np.abs(do_rows) * (p @ np.abs(v)), axis=1, keepdims=True)
    ds_err = (U + LSE_REL) * np.abs(ds) + p * ddelta
    return p, ds_err


def bwd_tolerance(q, k, v, dout, scale, causal, window, ref, row_block=512):
    """Tolerances (tQ, tK, tV) for the whole gradient, given ref = (dQ, dK, dV)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    bQ, bK, bV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, Lq, row_block):
                rows = np.arange(r0, min(Lq, r0 + row_block))
                vis = oracle.key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
                p, ds_err = _block_terms(q[b, rows, h], k[b, :, g], v[b, :, g], dout[b, rows, h],
                                         scale, vis)
                bQ[b, rows, h] = scale * ds_err @ np.abs(k[b, :, g])
                bK[b, :, g] += scale * ds_err.T @ np.abs(q[b, rows, h])
                bV[b, :, g] += (U + LSE_REL) * p.T @ np.abs(dout[b, rows, h])
    dQ, dK, dV = ref
    return tuple(2 * (bx + U * np.abs(rx)) + 1e-5 for bx, rx in ((bQ, dQ), (bK, dK), (bV, dV)))


def query_rows_tolerance(q, k, v, dout, b, h, rows, scale, causal, window, ref_rows):
    """Tolerance of dQ at selected rows of one (batch, query head)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    g = h // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    kk = _f64(k[b, :, g])
    vis = oracle.key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
    _, ds_err = _block_terms(_f64(q[b, rows, h]), kk, _f64(v[b, :, g]), _f64(dout[b, rows, h]),
                             scale, vis)
    return 2 * (scale * ds_err @ np.abs(kk) + U * np.abs(ref_rows)) + 1e-5


def key_rows_tolerance(q, k, v, dout, b, g, keys, scale, causal, window, ref_dk, ref_dv,
                       row_block=1024, row_start=0):
    """Tolerances of dK and dV at selected keys of one (batch, KV head)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    kk, vv = _f64(k[b, :, g]), _f64(v[b, :, g])
    bK = np.zeros((keys.size, d))
    bV = np.zeros((keys.size, v.shape[3]))
    for h in range(g * G, (g + 1) * G):
        for r0 in range(row_start, Lq, row_block):
            rows = np.arange(r0, min(Lq, r0 + row_block))
            vis = oracle.key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
            qr, dr = _f64(q[b, rows, h]), _f64(dout[b, rows, h])
            p, ds_err = _block_terms(qr, kk, vv, dr, scale, vis)
            bK += scale * ds_err[:, keys].T @ np.abs(qr)
            bV += (U + LSE_REL) * p[:, keys].T @ np.abs(dr)
    return (2 * (bK + U * np.abs(ref_dk)) + 1e-5, 2 * (bV + U * np.abs(ref_dv)) + 1e-5)


def ratio(got, ref, tol):
    """max |got - ref| / tol (<= 1 passes)."""
    got = _f64(got) if not isinstance(got, np.ndarray) or got.dtype == np.uint16 else got
    return float((np.abs(got - ref) / tol).max()) if ref.size else 0.0


def scale_default(d):
    return 1.0 / math.sqrt(d)
