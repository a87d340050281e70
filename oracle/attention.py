"""Plain float64 attention on the CPU (test infrastructure only; see package doc).

Nothing here is blocked, fused or reordered beyond what the definition
states: for each (batch, query head) the full score rows S are formed with a
matrix product, masked, exponentiated, normalised into P and multiplied by V.
Row blocks of at most ``row_block`` queries only bound memory; each block
still forms complete rows of S.
"""

import math

import numpy as np


def _f64(x):
    """Inputs as float64.  numpy has no bfloat16, so a uint16 array is read as
    bfloat16 bit patterns (exact: bf16 is the top half of an fp32)."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def key_visibility(Lq, Lk, causal, window_left=-1, window_right=-1, rows=None):
    """Boolean matrix vis[r, j]: is key j visible to query row rows[r]?

    Masking rules: the causal mask of autoregressive inference ("FlashAttention-3
    vs naive attention", sec. 1.1 and 2.1) and the sliding window
    ``window_size=(left, right)`` of the configuration skill page (sec. 3.3,
    where (4096, 0) means looking back 4096 tokens).  Readings taken where the
    pages are silent: query row i sits at absolute key position i + (Lk - Lq)
    (bottom-right alignment, so a one-token decode query sees its whole
    history); window bounds are inclusive; a negative side is unbounded.
    """
    i = np.arange(Lq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = i[:, None] + (Lk - Lq)
    j = np.arange(Lk, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], Lk), dtype=bool)
    if causal:
        vis &= j <= pos
    if window_left >= 0:
        vis &= j >= pos - window_left
    if window_right >= 0:
        vis &= j <= pos + window_right
    return vis


def attend_rows(q_rows, k, v, scale, vis, softcap=0.0, bias=None):
    """Standard attention for a block of query rows of one head.

    "FlashAttention-3 vs naive attention", sec. 1.1: S = scale * Q K^T (+mask),
    P = softmax(S), O = P V.  Softmax is the usual max-subtracted form (same
    page, sec. 6.1).  Returns O (n, dv), LSE (n,) with LSE = m + ln l, and P
    (n, Lk).  Rows with no visible key give O = 0, LSE = -inf, P = 0.

    Score modifiers ("flash-attention" skill page, sec. 3.3): softcap > 0
    replaces each logit x = scale * q.k by softcap * tanh(x / softcap); bias
    (n, Lk), e.g. ALiBi's, is then added.  Both come before the mask.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    s = scale * (q_rows @ k.T)                      # S, materialised
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])                 # masked entries -> exp(-inf) = 0
    l = e.sum(axis=1)
    ok = l > 0
    p = np.zeros_like(e)
    p[ok] = e[ok] / l[ok, None]                     # P, materialised
    lse = np.full(l.shape, -np.inf)
    lse[ok] = m_safe[ok] + np.log(l[ok])
    o = p @ v
    return o, lse, p


def alibi_bias(rows, Lq, Lk, slope):
    """ALiBi bias for query rows ``rows`` against keys 0..Lk-1 ("flash-attention"
    skill page, sec. 3.3: per-head alibi_slopes, used in place of RoPE).
    Reading taken (the page gives no formula): -slope * |i + (Lk - Lq) - j|,
    i.e. a penalty linear in the distance between the query's position
    (bottom-right alignment, as for the causal mask) and the key."""
    pos = np.asarray(rows, dtype=np.int64)[:, None] + (Lk - Lq)
    j = np.arange(Lk, dtype=np.int64)[None, :]
    return -float(slope) * np.abs(pos - j).astype(np.float64)


def _slope(alibi_slopes, b, h):
    """Slope of (batch b, query head h) from alibi_slopes of shape (Hq,) or (B, Hq)."""
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return a[h] if a.ndim == 1 else a[b, h]


def _kv_head(h, Hq, Hkv):
    """GQA/MQA broadcast ("flash-attention" skill page, appendix on GQA/MQA):
    Hkv divides Hq and query heads [g*G, (g+1)*G) share KV head g, G = Hq/Hkv
    (the repeat_kv / repeat_interleave convention)."""
    if Hq % Hkv != 0:
        raise ValueError("Hkv must divide Hq")
    return h // (Hq // Hkv)


def attention_rows_ref(q, k, v, b, h, rows, softmax_scale=None, causal=False,
                       window=(-1, -1), return_probs=False, softcap=0.0, alibi_slopes=None):
    """Selected query rows of one (batch b, query head h) of dense attention.

    q: (B, Lq, Hq, d); k, v: (B, Lk, Hkv, d).  Returns O (n, d), LSE (n,)
    (and P (n, Lk) if asked).  Used to check sampled rows at full size.
    """
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    vis = key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
    bias = None if alibi_slopes is None else alibi_bias(rows, Lq, Lk, _slope(alibi_slopes, b, h))
    o, lse, p = attend_rows(_f64(q[b, rows, h, :]), _f64(k[b, :, g, :]),
                            _f64(v[b, :, g, :]), scale, vis, softcap, bias)
    return (o, lse, p) if return_probs else (o, lse)


def attention_ref(q, k, v, softmax_scale=None, causal=False, window=(-1, -1),
                  row_block=1024, softcap=0.0, alibi_slopes=None):
    """Dense attention over (B, L, H, d) tensors, the layout of the skill
    page's flash_attn_func (sec. 3.1/3.2); default scale 1/sqrt(headdim).

    Returns O (B, Lq, Hq, d) float64 and LSE (B, Hq, Lq) float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Lk, Hkv, d) or v.shape[:3] != (B, Lk, Hkv):
        raise ValueError("q/k/v shapes disagree")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    O = np.zeros((B, Lq, Hq, v.shape[3]))
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kk, vv = k[b, :, g, :], v[b, :, g, :]
            for r0 in range(0, Lq, row_block):
                rows = np.arange(r0, min(Lq, r0 + row_block))
                vis = key_visibility(Lq, Lk, causal, window[0], window[1], rows=rows)
                bias = (None if alibi_slopes is None
                        else alibi_bias(rows, Lq, Lk, _slope(alibi_slopes, b, h)))
                o, lse, _ = attend_rows(q[b, rows, h, :], kk, vv, scale, vis, softcap, bias)
                O[b, rows, h, :] = o
                LSE[b, h, rows] = lse
    return O, LSE


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale=None,
                         causal=False, window=(-1, -1), row_block=1024, softcap=0.0,
                         alibi_slopes=None):
    """Packed variable-length attention (skill page sec. 3.4 and the appendix on
    continuous batching): sequences are concatenated along the token axis,
    cu_seqlens holds batch+1 cumulative offsets, and no token attends across
    sequences.  Each sequence is the dense definition on its own slice.

    q: (total_q, Hq, d); k, v: (total_k, Hkv, d).  Returns O (total_q, Hq, d)
    and LSE (Hq, total_q).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    Hq = q.shape[1]
    O = np.zeros((q.shape[0], Hq, v.shape[2]))
    LSE = np.full((Hq, q.shape[0]), -np.inf)
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe == qs:
            continue
        sl = None
        if alibi_slopes is not None:
            a = np.asarray(alibi_slopes, dtype=np.float64)
            sl = a if a.ndim == 1 else a[b]
        o, lse = attention_ref(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke],
                               softmax_scale, causal, window, row_block, softcap, sl)
        O[qs:qe] = o[0]
        LSE[:, qs:qe] = lse[0]
    return O, LSE


def gather_paged(cache, block_table_row, length, page_size):
    """Read the first ``length`` key rows of one sequence out of a paged cache.

    Paged KV ("flash-attention" skill page, appendix on PagedAttention, and the
    "FIA / FlashAttention" explainer, sec. 2): the cache is
    [num_pages, page_size, Hkv, d]; token j of the sequence lives in page
    block_table[j // page_size], slot j % page_size.
    """
    j = np.arange(length, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[j // page_size]
    return cache[pages, j % page_size]                # (length, Hkv, d)


def decode_paged_ref(q, k_cache, v_cache, block_table, cache_seqlens, page_size,
                     softmax_scale=None, window_left=-1, softcap=0.0, alibi_slopes=None):
    """One decode step over a paged KV cache ("flash-attention" skill page,
    appendix on PagedAttention / FlashDecoding; "FlashAttention-3 vs naive
    attention", sec. 2.2): each request's single query row attends to its
    cache_seqlens[b] cached tokens (all visible under bottom-right causal
    alignment; a left window keeps the last window_left + 1).  softcap and
    alibi_slopes ((Hq,) or (B, Hq)) are the score modifiers of attention_ref
    (skill page sec. 3.3, with the kvcache call's arguments); the query sits
    at position cache_seqlens[b] - 1.

    q: (B, 1, Hq, d); caches [num_pages, page_size, Hkv, d].  Returns
    O (B, 1, Hq, d) and LSE (B, Hq).
    """
    q = _f64(q)
    B, _, Hq, d = q.shape
    O = np.zeros((B, 1, Hq, d))   # caches may stay uint16 bf16 bits: only used rows convert
    LSE = np.zeros((B, Hq))
    for b in range(B):
        n = int(cache_seqlens[b])
        kk = _f64(gather_paged(k_cache, block_table[b], n, page_size))[None]
        vv = _f64(gather_paged(v_cache, block_table[b], n, page_size))[None]
        sl = None
        if alibi_slopes is not None:
            a = np.asarray(alibi_slopes, dtype=np.float64)
            sl = a if a.ndim == 1 else a[b]
        o, lse = attention_ref(q[b:b + 1], kk, vv, softmax_scale, causal=True,
                               window=(window_left, -1), softcap=softcap, alibi_slopes=sl)
        O[b] = o[0]
        LSE[b] = lse[0, :, 0]
    return O, LSE


def append_paged_ref(k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, page_size):
    """Write the K/V rows of new tokens into a paged cache ("flash-attention"
    skill page, sec. 3.5: k_new / v_new passed with cache_seqlens, each
    request's current cache length; appendix on PagedAttention for the page
    layout).  Reading taken where the page is silent: new token i of request b
    goes to sequence position cache_seqlens[b] + i, i.e. page
    block_table[b][pos // page_size], slot pos % page_size.

    k_new, v_new: (B, L_new, Hkv, d).  Returns new cache arrays; the inputs are
    not modified.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B, Ln = k_new.shape[:2]
    for b in range(B):
        pos = int(cache_seqlens[b]) + np.arange(Ln, dtype=np.int64)
        pages = np.asarray(block_table[b], dtype=np.int64)[pos // page_size]
        kc[pages, pos % page_size] = k_new[b]
        vc[pages, pos % page_size] = v_new[b]
    return kc, vc


def attention_kvcache_ref(q, k_cache, v_cache, block_table, cache_seqlens, page_size,
                          k_new=None, v_new=None, softmax_scale=None, causal=True,
                          window=(-1, -1), softcap=0.0, alibi_slopes=None):
    """Attention of several new query tokens over a paged KV cache (chunked
    prefill; "flash-attention" skill page, sec. 3.5 and the appendix on
    PagedAttention).  When k_new / v_new are given they are first appended at
    positions cache_seqlens[b] .. cache_seqlens[b] + Lq - 1 (append_paged_ref);
    request b then has n_b = cache_seqlens[b] (+ Lq when appending) keys, and
    its Lq query rows sit at the last Lq positions (bottom-right alignment, as
    for every Lq != Lk case here).

    q: (B, Lq, Hq, d).  Returns O (B, Lq, Hq, d), LSE (B, Hq, Lq) and the
    caches after the append (the given arrays when nothing is appended).
    """
    q = _f64(q)
    B, Lq, Hq, d = q.shape
    if k_new is not None:
        assert k_new.shape[1] == Lq and v_new.shape[1] == Lq
        k_cache, v_cache = append_paged_ref(k_cache, v_cache, k_new, v_new, block_table,
                                            cache_seqlens, page_size)
        extra = Lq
    else:
        extra = 0
    O = np.zeros((B, Lq, Hq, d))
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        n = int(cache_seqlens[b]) + extra
        kk = _f64(gather_paged(k_cache, block_table[b], n, page_size))[None]
        vv = _f64(gather_paged(v_cache, block_table[b], n, page_size))[None]
        sl = None
        if alibi_slopes is not None:
            a = np.asarray(alibi_slopes, dtype=np.float64)
            sl = a if a.ndim == 1 else a[b]
        o, lse = attention_ref(q[b:b + 1], kk, vv, softmax_scale, causal, window,
                               softcap=softcap, alibi_slopes=sl)
        O[b] = o[0]
        LSE[b] = lse[0]
    return O, LSE, k_cache, v_cache


def decode_split_partials_ref(q_row, k, v, scale, split_tokens, lo=0):
    """Split-KV partial results for one decode query row ("flash-attention"
    skill page, appendix on FlashDecoding / Split-KV: several workers take
    different KV ranges of the same head and the results are reduced).

    Keys [lo, len) are cut into chunks of ``split_tokens`` aligned to 0; each
    chunk is plain attention over its keys, giving (lse_s, O_s).
    """
    n = k.shape[0]
    lses, outs = [], []
    for s0 in range(0, n, split_tokens):
        ks = max(s0, lo)
        ke = min(n, s0 + split_tokens)
        if ke <= ks:
            continue
        vis = np.ones((1, ke - ks), dtype=bool)
        o, lse, _ = attend_rows(_f64(q_row)[None], k[ks:ke], v[ks:ke], scale, vis)
        lses.append(lse[0])
        outs.append(o[0])
    return np.array(lses), np.array(outs)


def merge_partials_ref(lse_parts, o_parts):
    """Reduce split partials into one row (the "online-softmax reduction" of the
    FIA explainer, sec. 2, and the final reduce of split-KV on the skill page).

    With M = max_s lse_s: LSE = M + ln sum_s exp(lse_s - M) and
    O = sum_s exp(lse_s - LSE) * O_s.  Empty input or all -inf gives (-inf, 0).
    """
    lse_parts = _f64(lse_parts)
    o_parts = _f64(o_parts)
    if lse_parts.size == 0 or not np.isfinite(lse_parts).any():
        dv = o_parts.shape[-1] if o_parts.ndim == 2 and o_parts.shape[-1] else 0
        return -np.inf, np.zeros(dv)
    M = lse_parts.max()
    w = np.exp(lse_parts - M)
    lse = M + math.log(w.sum())
    o = (np.exp(lse_parts - lse)[:, None] * o_parts).sum(axis=0)
    return lse, o


def online_softmax_ref(q_row, k, v, scale, block):
    """The streaming (online) softmax of the pages, written as its steps: keys
    are visited in blocks; a running row max m and normaliser l are kept; when
    a block raises the max, the old l and the output accumulator are rescaled by
    exp(m_old - m_new) ("FIA / FlashAttention" explainer, sec. 1; glossary page,
    "online normalization"; "FlashAttention-3 vs naive attention", sec. 6.2).

    Returns (O, LSE) for one query row; O is divided by l once at the end.
    """
    q_row, k, v = _f64(q_row), _f64(k), _f64(v)
    m = -np.inf
    l = 0.0
    acc = np.zeros(v.shape[1])
    for j0 in range(0, k.shape[0], block):
        s = scale * (k[j0:j0 + block] @ q_row)      # scores of this block
        m_new = max(m, s.max())
        alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ v[j0:j0 + block]
        m = m_new
    return acc / l, m + math.log(l)
