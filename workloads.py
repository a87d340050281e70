"""Seeded synthetic inputs for the attention workloads (no attention arithmetic).

This module only draws random numbers and lays them out.  Both sides use it:
the parity tests feed the same arrays to the HIP library and to the CPU
oracle, and bench.py times the library on them.  It imports neither of them.

Recipe (stated once, used everywhere):
  * rng = numpy.random.default_rng(seed) with seed = workload number (1..5);
  * normals are float32 ``rng.standard_normal`` rounded to bf16 with
    round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``);
  * arrays are drawn in the order listed per workload.

Shapes follow the pages' problem statement: dense Q/K/V are (B, L, H, d),
packed varlen tensors are (total_tokens, H, d) with cu_seqlens of length
batch+1, paged caches are [num_pages, page_size, Hkv, d] with a
[batch, max_blocks_per_seq] block table.
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def bf16_normal(rng, shape):
    """float32 N(0,1) draws rounded to bf16 (RNE); returns a CPU bf16 tensor."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


@dataclass
class Dense:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    causal: bool
    window: tuple
    scale: float


@dataclass
class Varlen:
    name: str
    q: torch.Tensor            # (total, H, d) bf16
    k: torch.Tensor
    v: torch.Tensor
    lens: np.ndarray           # per-sequence lengths, packing order
    cu_seqlens: np.ndarray     # (B+1,) int32
    causal: bool
    window: tuple
    scale: float

    @property
    def max_seqlen(self):
        return int(self.lens.max()) if len(self.lens) else 0


@dataclass
class Paged:
    name: str
    q: torch.Tensor            # (B, 1, Hq, d) bf16
    k_cache: torch.Tensor      # [num_pages, page_size, Hkv, d] bf16
    v_cache: torch.Tensor
    block_table: np.ndarray    # (B, max_blocks) int32
    seqlens: np.ndarray        # (B,) int32
    page_size: int
    split_tokens: int
    scale: float
    window_left: int = -1
    extra: dict = field(default_factory=dict)


# ---------------------------------------------------------------- workload 1
def small_dense(Hkv=1, seed=1):
    """Single head group, non-causal: B=1, Hq=2, L=128, d=64 (Hkv = 1 or 2)."""
    rng = np.random.default_rng(seed)
    q = bf16_normal(rng, (1, 128, 2, 64))
    k = bf16_normal(rng, (1, 128, Hkv, 64))
    v = bf16_normal(rng, (1, 128, Hkv, 64))
    return Dense(f"dense_b1_h2_kv{Hkv}_l128_d64_noncausal", q, k, v, False, (-1, -1), 1.0 / 8.0)


# ---------------------------------------------------------------- workload 2
def causal_mha(seed=2):
    """Causal MHA prefill: B=4, H=32, L=2048, d=128."""
    rng = np.random.default_rng(seed)
    shp = (4, 2048, 32, 128)
    q = bf16_normal(rng, shp)
    k = bf16_normal(rng, shp)
    v = bf16_normal(rng, shp)
    return Dense("causal_mha_b4_h32_l2048_d128", q, k, v, True, (-1, -1), 1.0 / math.sqrt(128))


# ---------------------------------------------------------------- workload 3
def causal_gqa_long(seed=3):
    """Long-context causal GQA prefill: B=1, Hq=32, Hkv=8, L=16384, d=128."""
    rng = np.random.default_rng(seed)
    q = bf16_normal(rng, (1, 16384, 32, 128))
    k = bf16_normal(rng, (1, 16384, 8, 128))
    v = bf16_normal(rng, (1, 16384, 8, 128))
    return Dense("causal_gqa_b1_hq32_hkv8_l16384_d128", q, k, v, True, (-1, -1),
                 1.0 / math.sqrt(128))


# ---------------------------------------------------------------- workload 4
def _decode_layout(rng, batch, page_size, pool_pages, len_lo, len_hi):
    """Lengths, page permutation and block table (the first draws of the
    paged-decode recipe)."""
    lens = rng.integers(len_lo, len_hi, size=batch, endpoint=True).astype(np.int32)
    perm = rng.permutation(pool_pages).astype(np.int32)
    max_blocks = -(-len_hi // page_size)
    npages = -(-lens.astype(np.int64) // page_size)
    used = int(npages.sum())
    if used >= pool_pages:
        raise ValueError("page pool too small")
    spare = int(perm[used])                       # first unassigned id: a NaN page
    table = np.full((batch, max_blocks), spare, dtype=np.int32)
    off = 0
    for b in range(batch):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    return lens, perm, table, npages, used, spare


def paged_decode_layout(seed=4, batch=64, page_size=16, pool_pages=40960, len_lo=512,
                        len_hi=8192):
    """The paged-decode workload's lengths and block table without its pools."""
    rng = np.random.default_rng(seed)
    lens, _, table, _, used, spare = _decode_layout(rng, batch, page_size, pool_pages,
                                                    len_lo, len_hi)
    return lens, table, used, spare


def paged_decode(seed=4, batch=64, Hq=32, Hkv=8, d=128, page_size=16, pool_pages=40960,
                 len_lo=512, len_hi=8192, split_tokens=512, chunk_pages=1024):
    """Paged-KV decode: 64 requests, q length 1, Hq=32, Hkv=8, d=128, contexts
    uniform in [512, 8192] (inclusive integers), 16-token pages taken from a
    40960-page pool in a seeded random permutation, 512-token splits.

    Draw order: lengths; page permutation; q; K pool; V pool (pools drawn in
    chunks of ``chunk_pages`` pages).  Request b takes the next
    ceil(len_b / page_size) ids of the permutation; unused block-table columns
    point at the first unassigned page.  Unassigned pages, and slots at or past
    a request's length in its last page, hold NaN: they must never influence a
    result.
    """
    rng = np.random.default_rng(seed)
    lens, perm, table, npages, used, spare = _decode_layout(
        rng, batch, page_size, pool_pages, len_lo, len_hi)
    q = bf16_normal(rng, (batch, 1, Hq, d))

    def pool():
        out = torch.empty((pool_pages, page_size, Hkv, d), dtype=torch.bfloat16)
        for p0 in range(0, pool_pages, chunk_pages):
            p1 = min(pool_pages, p0 + chunk_pages)
            out[p0:p1] = bf16_normal(rng, (p1 - p0, page_size, Hkv, d))
        return out

    kc = pool()
    vc = pool()
    assigned = np.zeros(pool_pages, dtype=bool)
    assigned[perm[:used]] = True
    nan = float("nan")
    kc[torch.from_numpy(~assigned)] = nan
    vc[torch.from_numpy(~assigned)] = nan
    for b in range(batch):
        tail = int(lens[b]) % page_size
        if tail:
            last = int(table[b, npages[b] - 1])
            kc[last, tail:] = nan
            vc[last, tail:] = nan
    return Paged("paged_decode_b64_hq32_hkv8_d128_p16", q, kc, vc, table, lens, page_size,
                 split_tokens, 1.0 / math.sqrt(d), -1,
                 {"pool_pages": pool_pages, "pages_used": used, "spare_page": spare})


# ---------------------------------------------------------------- workload 5
def _log_uniform_lengths(rng, nseq, lo, hi):
    return np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=nseq))).astype(np.int32)


def varlen_window_lengths(seed=5, nseq=16, lo=64, hi=8192):
    """The sequence lengths varlen_window draws (first draw of the same seed)."""
    return _log_uniform_lengths(np.random.default_rng(seed), nseq, lo, hi)


def varlen_window(seed=5, nseq=16, H=16, d=64, lo=64, hi=8192, window=(4096, 0)):
    """Varlen packed causal prefill with a sliding window: 16 sequences with
    lengths log-uniform in [64, 8192] (rint(exp(U(ln lo, ln hi)))), packed with
    cu_seqlens and no padding, H=16, d=64, window (4096, 0).
    Draw order: lengths; q; k; v."""
    rng = np.random.default_rng(seed)
    lens = _log_uniform_lengths(rng, nseq, lo, hi)
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = bf16_normal(rng, (T, H, d))
    k = bf16_normal(rng, (T, H, d))
    v = bf16_normal(rng, (T, H, d))
    return Varlen("varlen_causal_window4096_h16_d64", q, k, v, lens, cu, True, window,
                  1.0 / math.sqrt(d))


# ------------------------------------------------------- maximum sizes
def device_normal(seed, shape, device="cuda"):
    """N(0, 1) rounded to bf16, drawn on `device` by torch's generator seeded
    with `seed` (fp32 normals, then RNE to bf16).  Used where numpy would be
    too slow (tensors of 2^30 elements); tests copy the same tensor to the host
    for the oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


# ------------------------------------------------------- backward inputs
def upstream_grad(seed, shape):
    """Upstream gradient dO for the backward pass: N(0, 1) rounded to bf16
    (same recipe as q, k, v), drawn from its own seed."""
    return bf16_normal(np.random.default_rng(seed), shape)


# ------------------------------------------------------------ small helpers
def random_dense(seed, B, Lq, Lk, Hq, Hkv, d, causal=False, window=(-1, -1), scale=None):
    """Small dense case for parity sweeps (same recipe, arbitrary shape)."""
    rng = np.random.default_rng(seed)
    q = bf16_normal(rng, (B, Lq, Hq, d))
    k = bf16_normal(rng, (B, Lk, Hkv, d))
    v = bf16_normal(rng, (B, Lk, Hkv, d))
    return Dense(f"dense_s{seed}", q, k, v, causal, window,
                 (1.0 / math.sqrt(d)) if scale is None else scale)


def random_varlen(seed, lens, Hq, Hkv, d, causal=True, window=(-1, -1)):
    """Small varlen case with given lengths (packing order as given)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = bf16_normal(rng, (T, Hq, d))
    k = bf16_normal(rng, (T, Hkv, d))
    v = bf16_normal(rng, (T, Hkv, d))
    return Varlen(f"varlen_s{seed}", q, k, v, lens, cu, causal, window, 1.0 / math.sqrt(d))


def random_varlen_qk(seed, lens_q, lens_k, Hq, Hkv, d):
    """Small varlen case with separate query and key lengths per sequence.
    Returns (q, k, v, cu_q, cu_k); draw order q, k, v."""
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = bf16_normal(rng, (int(cu_q[-1]), Hq, d))
    k = bf16_normal(rng, (int(cu_k[-1]), Hkv, d))
    v = bf16_normal(rng, (int(cu_k[-1]), Hkv, d))
    return q, k, v, cu_q, cu_k


def random_paged(seed, lens, Hq, Hkv, d, page_size, pool_pages, split_tokens=512,
                 max_blocks=None, window_left=-1):
    """Small paged case with the same layout rules as ``paged_decode``."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    npages = -(-lens.astype(np.int64) // page_size)
    if max_blocks is None:
        max_blocks = int(max(1, npages.max()))
    perm = rng.permutation(pool_pages).astype(np.int32)
    used = int(npages.sum())
    if used >= pool_pages:
        raise ValueError("page pool too small")
    spare = int(perm[used])
    table = np.full((len(lens), max_blocks), spare, dtype=np.int32)
    off = 0
    for b in range(len(lens)):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    q = bf16_normal(rng, (len(lens), 1, Hq, d))
    kc = bf16_normal(rng, (pool_pages, page_size, Hkv, d))
    vc = bf16_normal(rng, (pool_pages, page_size, Hkv, d))
    assigned = np.zeros(pool_pages, dtype=bool)
    assigned[perm[:used]] = True
    kc[torch.from_numpy(~assigned)] = float("nan")
    vc[torch.from_numpy(~assigned)] = float("nan")
    for b in range(len(lens)):
        tail = int(lens[b]) % page_size
        if tail and npages[b]:
            last = int(table[b, npages[b] - 1])
            kc[last, tail:] = float("nan")
            vc[last, tail:] = float("nan")
    return Paged(f"paged_s{seed}", q, kc, vc, table, lens, page_size, split_tokens,
                 1.0 / math.sqrt(d), window_left, {"spare_page": spare})


@dataclass
class KVCache:
    """Chunked prefill over a paged cache: q (B, Lq, Hq, d); caches
    [num_pages, page_size, Hkv, d]; cache_seqlens = keys already cached;
    k_new / v_new (B, Lq, Hkv, d) or None."""
    name: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_new: object
    v_new: object
    block_table: np.ndarray
    cache_seqlens: np.ndarray
    page_size: int
    scale: float
    causal: bool
    window: tuple


def random_kvcache(seed, lens, Lq, Hq, Hkv, d, page_size, append=True, causal=True,
                   window=(-1, -1), spare_pages=3):
    """Paged cache holding lens[b] tokens per request, plus (when appending)
    pages already allocated for the Lq new tokens.  Draw order: page
    permutation, q, K pool, V pool, k_new, v_new.  Unassigned pages and slots
    at or past each request's final length are NaN, so a wrong read shows."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    total = lens.astype(np.int64) + (Lq if append else 0)
    npages = -(-total // page_size)
    pool = int(npages.sum()) + spare_pages
    max_blocks = int(max(1, npages.max()))
    perm = rng.permutation(pool).astype(np.int32)
    spare = int(perm[int(npages.sum())])
    table = np.full((len(lens), max_blocks), spare, dtype=np.int32)
    off = 0
    for b in range(len(lens)):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    q = bf16_normal(rng, (len(lens), Lq, Hq, d))
    kc = bf16_normal(rng, (pool, page_size, Hkv, d))
    vc = bf16_normal(rng, (pool, page_size, Hkv, d))
    assigned = np.zeros(pool, dtype=bool)
    assigned[perm[:int(npages.sum())]] = True
    kc[torch.from_numpy(~assigned)] = float("nan")
    vc[torch.from_numpy(~assigned)] = float("nan")
    for b in range(len(lens)):
        # slots from the cached length on are NaN until the append fills them
        for pos in range(int(lens[b]), int(npages[b]) * page_size):
            pg = int(table[b, pos // page_size])
            kc[pg, pos % page_size] = float("nan")
            vc[pg, pos % page_size] = float("nan")
    kn = vn = None
    if append:
        kn = bf16_normal(rng, (len(lens), Lq, Hkv, d))
        vn = bf16_normal(rng, (len(lens), Lq, Hkv, d))
    return KVCache(f"kvcache_s{seed}", q, kc, vc, kn, vn, table, lens, page_size,
                   1.0 / math.sqrt(d), causal, window)


def chunked_prefill(seed=6):
    """A chunk of 512 new tokens per request appended to, and attending over,
    a paged cache of 2048..6144 cached tokens: 4 requests, Hq=32, Hkv=8,
    d=128, 16-token pages, causal.  Cache lengths are drawn first."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(2048, 6144, 4, endpoint=True).astype(np.int32)
    w = random_kvcache(seed + 1000, lens, 512, 32, 8, 128, 16, append=True)
    w.name = "chunked_prefill_b4_lq512_h32_kv8_d128_p16"
    return w
