"""Elementwise error bounds for the backward kernels (test helper, not collected).

The bound follows the arithmetic of the HIP path, to first order in the bf16
unit roundoff u = 2^-8 (round to nearest even, 8 significant bits).  Each
error source is either systematic along the sum it enters (the same factor
for every term, bounded with the triangle inequality) or an independent
rounding per term (bounded by C_RND times the root of the sum of squares of
the terms' worst cases, C_RND = 4, about seven standard deviations of a
rounding error spread evenly over [-u, u]):

  * P is recomputed in fp32 from bf16 Q, K and the forward's fp32 LSE: a
    relative error of at most 1e-4 that is the same for a whole query row,
    so it scales row i of dS, and so dQ_i, by (1 + e_i): |e_i| <= 1e-4.
  * delta_i = dO_i . O_i uses the forward's bf16 O.  O_id errs by its bf16
    P (one rounding per key j, shared by every d) and by its own rounding
    (one per d), so delta_i errs by at most
        dd_i = C_RND u (sqrt(sum_j (P_ij dP_ij)^2) + sqrt(sum_d (dO_id O_id)^2)),
    the same for the whole row: it moves dQ_i by scale dd_i |(P K)_i|.
  * dS = P (dP - delta) is rounded to bf16 (one rounding per element).
  * dV = P^T dO takes P rounded to bf16 (one rounding per element).
  * dQ = scale dS K, dK = scale dS^T Q, dV accumulate in fp32 and are
    rounded to bf16 on output (u |g|).

So, per element (the sums for dK and dV also run over the query heads of a
KV group; the per-row errors of different rows are bounded linearly there):
  |dQ_id err| <= 1e-4 |dQ_id| + scale dd_i |(P K)_id|
                 + C_RND u scale sqrt(sum_j dS_ij^2 K_jd^2) + u |dQ_id|
  |dK_jd err| <= scale sum_i (1e-4 |dS_ij| + P_ij dd_i) |Q_id|
                 + C_RND u scale sqrt(sum_i dS_ij^2 Q_id^2) + u |dK_jd|
  |dV_jd err| <= 1e-4 sum_i P_ij |dO_id| + C_RND u sqrt(sum_i P_ij^2 dO_id^2) + u |dV_jd|
The tests allow twice this bound plus 1e-5 (fp32 accumulation order, outputs
that are 0).  P, O, dP, dS and delta come from the float64 oracle.
"""

import math

import numpy as np

import oracle

U = 2.0 ** -8
LSE_REL = 1e-4
C_RND = 4.0


def _f64(x):
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _block_terms(q_rows, k, v, do_rows, scale, vis):
    """P, dS and the delta error bound dd (one per row) for one block of query
    rows of one head."""
    o, _, p = oracle.attend_rows(q_rows, k, v, scale, vis)
    dp = do_rows @ v.T
    D = np.sum(do_rows * o, axis=1, keepdims=True)
    ds = p * (dp - D)
    dd = C_RND * U * (np.sqrt(np.sum((p * dp) ** 2, axis=1, keepdims=True))
                      + np.sqrt(np.sum((do_rows * o) ** 2, axis=1, keepdims=True)))
    return p, ds, dd


def _dq_terms(p, ds, dd, k, scale):
    """The parts of the dQ bound that do not scale with dQ itself."""
    return scale * (dd * np.abs(p @ k) + C_RND * U * np.sqrt((ds ** 2) @ (k ** 2)))


def _dq_tolerance(part, dq_ref):
    return 2 * (part + (LSE_REL + U) * np.abs(dq_ref)) + 1e-5


class _KeySums:
    """Accumulates the dK / dV bound terms of some keys over query rows and heads."""

    def __init__(self, shape_k, shape_v):
        self.lin_k, self.sq_k = np.zeros(shape_k), np.zeros(shape_k)
        self.lin_v, self.sq_v = np.zeros(shape_v), np.zeros(shape_v)

    def add(self, p, ds, dd, q_rows, do_rows, scale):
        self.lin_k += scale * (LSE_REL * np.abs(ds) + p * dd).T @ np.abs(q_rows)
        self.sq_k += scale ** 2 * (ds ** 2).T @ (q_rows ** 2)
        self.lin_v += LSE_REL * p.T @ np.abs(do_rows)
        self.sq_v += (p ** 2).T @ (do_rows ** 2)

    def tolerances(self, dk_ref, dv_ref):
        tk = 2 * (self.lin_k + C_RND * U * np.sqrt(self.sq_k) + U * np.abs(dk_ref)) + 1e-5
        tv = 2 * (self.lin_v + C_RND * U * np.sqrt(self.sq_v) + U * np.abs(dv_ref)) + 1e-5
        return tk, tv


def bwd_tolerance(q, k, v, dout, scale, causal, window, ref, row_block=512):
    """Tolerances (tQ, tK, tV) for the whole gradient, given ref = (dQ, dK, dV)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    dQ, dK, dV = ref
    tQ, tK, tV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for g in range(Hkv):
            sums = _KeySums((Lk, d), (Lk, v.shape[3]))
            for h in range(g * G, (g + 1) * G):
                for r0 in range(0, Lq, row_block):
                    rows = np.arange(r0, min(Lq, r0 + row_block))
                    vis = oracle.key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
                    p, ds, dd = _block_terms(q[b, rows, h], k[b, :, g], v[b, :, g], dout[b, rows, h],
                                             scale, vis)
                    tQ[b, rows, h] = _dq_tolerance(_dq_terms(p, ds, dd, k[b, :, g], scale), dQ[b, rows, h])
                    sums.add(p, ds, dd, q[b, rows, h], dout[b, rows, h], scale)
            tK[b, :, g], tV[b, :, g] = sums.tolerances(dK[b, :, g], dV[b, :, g])
    return tQ, tK, tV


def query_rows_tolerance(q, k, v, dout, b, h, rows, scale, causal, window, ref_rows):
    """Tolerance of dQ at selected rows of one (batch, query head)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    g = h // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    kk = _f64(k[b, :, g])
    vis = oracle.key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
    p, ds, dd = _block_terms(_f64(q[b, rows, h]), kk, _f64(v[b, :, g]), _f64(dout[b, rows, h]),
                             scale, vis)
    return _dq_tolerance(_dq_terms(p, ds, dd, kk, scale), ref_rows)


def key_rows_tolerance(q, k, v, dout, b, g, keys, scale, causal, window, ref_dk, ref_dv,
                       row_block=1024, row_start=0):
    """Tolerances of dK and dV at selected keys of one (batch, KV head)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    kk, vv = _f64(k[b, :, g]), _f64(v[b, :, g])
    sums = _KeySums((keys.size, d), (keys.size, v.shape[3]))
    for h in range(g * G, (g + 1) * G):
        for r0 in range(row_start, Lq, row_block):
            rows = np.arange(r0, min(Lq, r0 + row_block))
            vis = oracle.key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
            qr, dr = _f64(q[b, rows, h]), _f64(dout[b, rows, h])
            p, ds, dd = _block_terms(qr, kk, vv, dr, scale, vis)
            sums.add(p[:, keys], ds[:, keys], dd, qr, dr, scale)
    return sums.tolerances(ref_dk, ref_dv)


def ratio(got, ref, tol):
    """max |got - ref| / tol (<= 1 passes)."""
    got = _f64(got) if not isinstance(got, np.ndarray) or got.dtype == np.uint16 else got
    return float((np.abs(got - ref) / tol).max()) if ref.size else 0.0


def scale_default(d):
    return 1.0 / math.sqrt(d)
