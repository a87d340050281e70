"""GPU parity: the HIP library (through the C ABI) against the CPU fp64 oracle.

Small cases are compared element by element over every output; they span
several 128-row / 64-key tiles with ragged tails and cover each mask mode,
MHA/GQA/MQA, both head dims, Lq != Lk, fully masked rows, zero-length varlen
sequences, plans in heaviest-first, shuffled and partial order, and paged
layouts with several page sizes and split sizes.  The five
named workloads run at full size in the launch configuration bench.py times,
with outputs NaN-poisoned before the call, and every output element of each is
compared with the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bits, check, dev, f64, nan_like, oracle_rows_parallel

pytestmark = pytest.mark.gpu


def run_dense(fa, w):
    o, lse = fa.fa_fwd(dev(w.q), dev(w.k), dev(w.v), w.scale, w.causal, w.window)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


# --------------------------------------------------------------- small dense
@pytest.mark.parametrize("Hkv", [1, 2])
def test_small_dense_workload(fa, Hkv):
    w = workloads.small_dense(Hkv=Hkv)
    o, lse = run_dense(fa, w)
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), w.scale, w.causal, w.window)
    check(w.name, o, lse, O, LSE)


DENSE_CASES = [
    # B, Lq, Lk, Hq, Hkv, d, causal, window
    (2, 300, 300, 4, 2, 128, True, (-1, -1)),
    (2, 300, 300, 4, 4, 64, False, (-1, -1)),
    (1, 257, 257, 8, 1, 128, True, (37, 0)),
    (1, 200, 200, 2, 2, 64, False, (50, 20)),
    (1, 129, 385, 2, 1, 128, True, (-1, -1)),      # Lq < Lk: bottom-right causal
    (1, 385, 129, 2, 2, 64, True, (-1, -1)),       # Lq > Lk: first rows see no key
    (3, 64, 64, 2, 2, 128, False, (-1, 5)),        # right-only window
    (1, 1, 77, 4, 2, 128, True, (-1, -1)),         # a single query row
    (1, 1000, 1000, 2, 1, 64, True, (100, 0)),
    (1, 33, 1, 2, 1, 64, False, (-1, -1)),         # one key
    (2, 190, 190, 6, 3, 128, True, (0, 0)),        # window (0, 0): self only
    (1, 160, 160, 4, 2, 64, False, (-1, -1)),
    # odd key-tile counts whose extra (padding) tile holds real keys no row
    # sees (most of the workgroups of these shapes)
    (1, 640, 640, 2, 1, 128, False, (100, 30)),
    (1, 900, 900, 4, 2, 128, True, (40, 0)),
    (1, 900, 900, 2, 2, 64, True, (10, 0)),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "-".join(map(str, c[:6])) + f"-c{int(c[6])}-w{c[7][0]}_{c[7][1]}")
def test_dense_sweep(fa, case):
    B, Lq, Lk, Hq, Hkv, d, causal, window = case
    w = workloads.random_dense(100 + Lq + Lk + d + Hq, B, Lq, Lk, Hq, Hkv, d, causal, window)
    o, lse = run_dense(fa, w)
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), w.scale, causal, window)
    check(f"dense{case}", o, lse, O, LSE)


@pytest.mark.parametrize("d", [64, 128])
def test_dense_rescale_stress(fa, d):
    """Scores that rise along the keys force the running max up on every tile."""
    B, L, H = 1, 512, 2
    w = workloads.random_dense(77, B, L, L, H, H, d, True)
    k = w.k.float()
    qdir = w.q.float()[:, -1:, :, :] / w.q.float()[:, -1:, :, :].norm(dim=-1, keepdim=True)
    ramp = torch.linspace(0, 24, L).view(1, L, 1, 1)
    w.k = (k + ramp * qdir).to(torch.bfloat16)
    o, lse = run_dense(fa, w)
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), w.scale, True)
    check("rescale_stress", o, lse, O, LSE)


def test_dense_large_scale_values(fa):
    """A large softmax scale makes P nearly one-hot; checks the max/exponent path."""
    w = workloads.random_dense(78, 1, 256, 256, 2, 1, 64, True, scale=2.0)
    o, lse = run_dense(fa, w)
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), 2.0, True)
    check("large_scale", o, lse, O, LSE)


def test_huge_windows_equal_unbounded(fa):
    """A window side of 2^31 - 1 reaches every key: results must equal the
    unbounded side bit for bit (regression: the kernels' row + window sums
    must not overflow)."""
    big = 2 ** 31 - 1
    w = workloads.random_dense(79, 2, 200, 300, 4, 2, 128, False)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    for causal, win, ref_win in [(False, (big, big), (-1, -1)), (True, (big, -1), (-1, -1)),
                                 (False, (big, 5), (-1, 5)), (False, (7, big), (7, -1))]:
        o1, l1 = fa.fa_fwd(q, k, v, w.scale, causal, win)
        o2, l2 = fa.fa_fwd(q, k, v, w.scale, causal, ref_win)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (causal, win)
        assert torch.equal(l1, l2)
    o, lse = fa.fa_fwd(q, k, v, w.scale, False, (big, big))
    torch.cuda.synchronize()
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), w.scale, False, (big, big))
    check("huge window", o.cpu(), lse.cpu(), O, LSE)
    p = workloads.random_paged(80, [300, 40], 8, 2, 128, 16, 30, 128, max_blocks=24)
    a = run_decode(fa, p, window_left=big)
    b = run_decode(fa, p, window_left=-1)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


# -------------------------------------------------------------------- varlen
VARLEN_CASES = [
    ([1, 0, 7, 128, 129, 300], 4, 2, 128, True, (-1, -1)),
    ([1, 0, 7, 128, 129, 300], 4, 4, 64, True, (50, 0)),
    ([250, 3, 64], 2, 1, 64, False, (-1, -1)),
    ([513, 17], 8, 8, 128, False, (30, 30)),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{len(c[0])}-h{c[1]}-kv{c[2]}-d{c[3]}-c{int(c[4])}-w{c[5][0]}")
def test_varlen_sweep(fa, case):
    lens, Hq, Hkv, d, causal, window = case
    w = workloads.random_varlen(200 + sum(lens) + d, lens, Hq, Hkv, d, causal, window)
    cu = dev(torch.from_numpy(w.cu_seqlens))
    o, lse = fa.fa_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), cu, cu, w.max_seqlen, w.max_seqlen,
                              w.scale, causal, window)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_varlen_ref(bits(w.q), bits(w.k), bits(w.v), w.cu_seqlens,
                                         w.cu_seqlens, w.scale, causal, window)
    check(f"varlen{case}", o.cpu(), lse.cpu(), O, LSE)



VARLEN_QK_CASES = [
    # query lengths, key lengths, Hq, Hkv, d, causal, window
    ([100, 0, 260, 7], [300, 50, 260, 1], 4, 2, 128, True, (-1, -1)),   # chunks over longer prefixes; no rows
    ([300, 40, 129], [0, 400, 64], 4, 1, 64, True, (64, -1)),           # no keys; Lq > Lk
    ([65, 200], [900, 333], 8, 8, 128, False, (100, 20)),                # two-sided window, Lq < Lk
    ([128, 1], [1000, 1], 2, 2, 64, True, (0, 0)),                       # self only
]


@pytest.mark.parametrize("case", VARLEN_QK_CASES, ids=lambda c: f"n{len(c[0])}-h{c[2]}-kv{c[3]}-d{c[4]}-c{int(c[5])}-w{c[6][0]}_{c[6][1]}")
def test_varlen_separate_query_key_lengths(fa, case):
    """Packed sequences whose query and key counts differ (cu_seqlens_q != cu_seqlens_k):
    the causal mask aligns each sequence's last query with its last key."""
    lq, lk, Hq, Hkv, d, causal, window = case
    q, k, v, cq, ck = workloads.random_varlen_qk(1300 + sum(lq) + sum(lk) + d, lq, lk, Hq, Hkv, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fa_fwd_varlen(dev(q), dev(k), dev(v), dev(torch.from_numpy(cq)), dev(torch.from_numpy(ck)),
                              max(lq), max(lk), scale, causal, window)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_varlen_ref(bits(q), bits(k), bits(v), cq, ck, scale, causal, window)
    check(f"varlen_qk{case}", o.cpu(), lse.cpu(), O, LSE)
    # the planned run over the same batch gives the same bits
    plan = dev(torch.from_numpy(np.ascontiguousarray(fa.fa_varlen_plan(cq, ck, causal, window))))
    o2, lse2 = fa.fa_fwd_varlen_run(dev(q), dev(k), dev(v), dev(torch.from_numpy(cq)),
                                    dev(torch.from_numpy(ck)), plan, max(lq), max(lk), scale, causal, window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)

# -------------------------------------------------------------------- decode
def run_decode(fa, w, split=None, window_left=None):
    out = fa.fa_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache),
                             dev(torch.from_numpy(w.block_table)), dev(torch.from_numpy(w.seqlens)),
                             w.scale, w.window_left if window_left is None else window_left,
                             w.split_tokens if split is None else split)
    torch.cuda.synchronize()
    return out[0].cpu(), out[1].cpu()


def decode_ref(w, window_left=None):
    return oracle.decode_paged_ref(bits(w.q), bits(w.k_cache), bits(w.v_cache), w.block_table,
                                   w.seqlens, w.page_size, w.scale,
                                   w.window_left if window_left is None else window_left)


DECODE_CASES = [
    # lens, Hq, Hkv, d, page_size, split, window_left
    ([1, 15, 16, 17, 511, 512, 513, 1000], 8, 2, 128, 16, 512, -1),
    ([1, 15, 16, 17, 511, 512, 513, 1000], 8, 2, 128, 16, 16, -1),
    ([300, 64, 900], 4, 4, 64, 16, 0, -1),
    ([300, 7, 900], 8, 1, 128, 8, 128, -1),        # MQA, page_size 8 (< 16)
    ([333, 1, 64], 4, 2, 128, 1, 64, -1),          # page_size 1
    ([300, 7, 900], 16, 2, 128, 8, 128, -1),       # general kernel, 8-row subgroups
    ([1000, 50], 16, 2, 64, 8, 256, 300),          # the same at d = 64, window
    ([700, 129], 32, 2, 128, 32, 256, -1),         # 16 heads per KV head: two subgroups of 8
    ([1000, 50], 6, 2, 64, 16, 512, 100),          # 3 heads per KV head, window
    ([0, 40], 4, 2, 128, 16, 512, -1),             # an empty cache
    # four KV heads per workgroup (d = 128, <= 4 heads per KV head, 16 | page_size)
    ([1, 15, 16, 17, 511, 512, 513, 1000], 32, 8, 128, 16, 512, -1),
    ([700, 33, 129], 8, 8, 128, 16, 64, -1),       # MHA: one query per KV head
    ([1000, 50, 3], 12, 4, 128, 32, 256, 100),     # 3 heads per KV head, window
    ([517, 0, 77], 8, 4, 128, 16, 16, 37),         # 2 heads per KV head, 16-token splits
    # two KV heads per workgroup (d = 128, 5 to 8 heads per KV head, 16 | page_size)
    ([1, 15, 16, 17, 511, 512, 513, 1000], 16, 2, 128, 16, 512, -1),
    ([1000, 50, 3], 12, 2, 128, 32, 256, 100),     # 6 heads per KV head, window
    ([517, 0, 77, 33], 28, 4, 128, 16, 16, -1),    # 7 heads per KV head, 16-token splits
    ([300, 7, 900], 8, 1, 128, 16, 128, -1),       # 8 heads, one KV head: general kernel
    # d = 64 head sets: two tokens per load (NH = 4), four tokens per load (NH = 2)
    ([1, 15, 16, 17, 511, 512, 513, 1000], 16, 4, 64, 16, 512, -1),
    ([700, 33, 129], 16, 2, 64, 32, 64, 100),      # 8 heads per KV head, window
    ([517, 0, 77], 20, 4, 64, 16, 16, -1),         # 5 heads per KV head, 16-token splits
    # more than 8 heads per KV head: two-head sets in query subgroups of 8
    ([1000, 50, 3], 48, 4, 64, 16, 512, 100),      # 12 heads per KV head (4 in the last)
    ([700, 33, 129], 40, 2, 128, 16, 256, -1),     # 20 heads per KV head: three subgroups
    # odd Hkv: the general kernel (one scalar page id per 16-key block)
    ([300, 7, 900], 16, 1, 128, 16, 128, -1),      # 16 heads, one KV head
    ([517, 0, 77], 60, 3, 64, 32, 64, 200),        # 20 heads per KV head, window
    ([700, 129], 12, 3, 128, 16, 512, -1),         # 4 heads per KV head, Hkv = 3
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"n{len(c[0])}-h{c[1]}-kv{c[2]}-d{c[3]}-p{c[4]}-s{c[5]}-w{c[6]}")
def test_decode_sweep(fa, case):
    lens, Hq, Hkv, d, ps, split, wl = case
    npages = sum(-(-l // ps) for l in lens) + 3
    w = workloads.random_paged(300 + sum(lens) + ps, lens, Hq, Hkv, d, ps, npages, split,
                               max_blocks=max(1, -(-max(lens) // ps)) + 2, window_left=wl)
    o, lse = run_decode(fa, w)
    O, LSE = decode_ref(w)
    check(f"decode{case}", o, lse, O, LSE)


@pytest.mark.parametrize("case", [
    # lens, Hq, Hkv, d, page_size, split: head sets of four and two KV heads, then the
    # general kernel (page size 8)
    ([3000, 700, 1500], 32, 8, 128, 16, 512),
    ([3000, 700, 1500], 64, 8, 128, 16, 512),
    ([3000, 700, 1500], 32, 8, 64, 16, 512),
    ([3000, 700, 1500], 64, 8, 64, 16, 512),
    ([3000, 700, 1500], 128, 8, 128, 16, 512),
    ([3000, 700, 1500], 8, 2, 128, 16, 512),
    ([2000, 333], 8, 2, 64, 8, 256),
])
def test_decode_rescale_stress(fa, case):
    """K rows gain a component along the request's mean query that grows with
    the position, so the running max rises chunk after chunk (the rescale
    branch of the split kernels), planned and unplanned."""
    lens, Hq, Hkv, d, ps, split = case
    npages = sum(-(-l // ps) for l in lens) + 3
    w = workloads.random_paged(500 + Hq + d, lens, Hq, Hkv, d, ps, npages, split)
    G = Hq // Hkv
    kc = w.k_cache.float()
    for b, n in enumerate(lens):
        q = w.q[b, 0].float().view(Hkv, G, d).mean(dim=1)            # (Hkv, d)
        qdir = q / q.norm(dim=-1, keepdim=True)
        for j in range(n):
            kc[w.block_table[b, j // ps], j % ps] += (200.0 * j / n) * qdir
    w.k_cache = kc.to(torch.bfloat16)
    # the input does what it is for: within a split, some 16-key chunk's max
    # score exceeds the split's first chunk's by more than 2^8 (log2 units)
    b, n = 0, lens[0]
    keys = torch.stack([w.k_cache[w.block_table[b, j // ps], j % ps].float() for j in range(n)])
    s2 = torch.einsum("jgd,gxd->jgx", keys, w.q[b, 0].float().view(Hkv, G, d)) * (w.scale / math.log(2))
    cmax = s2[: n // 16 * 16].reshape(n // 16, 16, -1).amax(dim=(1, 2))
    per = split // 16
    assert any((cmax[i + 1:i + per] - cmax[i]).max() > 8 for i in range(0, len(cmax) - per, per))
    O, LSE = decode_ref(w)
    o, lse = run_decode(fa, w)
    check(f"decode rescale{case}", o, lse, O, LSE)
    o2, lse2 = run_decode_planned(fa, w)
    check(f"decode rescale planned{case}", o2, lse2, O, LSE)


def run_decode_planned(fa, w, plan=None):
    max_blocks = w.block_table.shape[1]
    if plan is None:
        plan = fa.fa_decode_plan(w.seqlens, w.page_size, max_blocks, w.window_left, w.split_tokens)
    out = fa.fa_decode_paged_run(dev(w.q), dev(w.k_cache), dev(w.v_cache),
                                 dev(torch.from_numpy(w.block_table)),
                                 dev(torch.from_numpy(w.seqlens)),
                                 dev(torch.from_numpy(np.ascontiguousarray(plan).reshape(-1, 2))),
                                 w.scale, w.window_left, w.split_tokens)
    torch.cuda.synchronize()
    return out[0].cpu(), out[1].cpu()


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"n{len(c[0])}-h{c[1]}-kv{c[2]}-d{c[3]}-p{c[4]}-s{c[5]}-w{c[6]}")
def test_decode_run_sweep(fa, case):
    lens, Hq, Hkv, d, ps, split, wl = case
    npages = sum(-(-l // ps) for l in lens) + 3
    w = workloads.random_paged(300 + sum(lens) + ps, lens, Hq, Hkv, d, ps, npages, split,
                               max_blocks=max(1, -(-max(lens) // ps)) + 2, window_left=wl)
    o, lse = run_decode_planned(fa, w)
    O, LSE = decode_ref(w)
    check(f"decode run{case}", o, lse, O, LSE)
    o2, lse2 = run_decode(fa, w)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


def test_decode_run_any_order_and_empty_plan(fa):
    w = workloads.random_paged(977, [1000, 3, 513], 8, 2, 128, 16, 200, 256, max_blocks=70)
    plan = fa.fa_decode_plan(w.seqlens, 16, 70, -1, 256)
    ref = run_decode_planned(fa, w, plan)
    shuffled = plan[np.random.default_rng(3).permutation(len(plan))]
    o, lse = run_decode_planned(fa, w, shuffled)
    assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)) and torch.equal(lse, ref[1])
    # every request empty: the plan has no item and the merge alone writes O = 0, LSE = -inf
    e = workloads.random_paged(978, [0, 0], 4, 2, 128, 16, 8, 512, max_blocks=4)
    plan = fa.fa_decode_plan(e.seqlens, 16, 4, -1, 512)
    assert plan.shape == (0, 2)
    o, lse = run_decode_planned(fa, e, plan)
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


# ------------------------------------------------- varlen plan / run split
def run_planned(fa, w, plan=None, out=None, lse=None):
    if plan is None:
        plan = fa.fa_varlen_plan(w.cu_seqlens, w.cu_seqlens, w.causal, w.window)
    cu = dev(torch.from_numpy(w.cu_seqlens))
    o, l = fa.fa_fwd_varlen_run(dev(w.q), dev(w.k), dev(w.v), cu, cu,
                                dev(torch.from_numpy(np.ascontiguousarray(plan))),
                                w.max_seqlen, w.max_seqlen, w.scale, w.causal, w.window,
                                out=out, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{len(c[0])}-h{c[1]}-kv{c[2]}-d{c[3]}-c{int(c[4])}-w{c[5][0]}")
def test_varlen_run_sweep(fa, case):
    lens, Hq, Hkv, d, causal, window = case
    w = workloads.random_varlen(200 + sum(lens) + d, lens, Hq, Hkv, d, causal, window)
    o, lse = run_planned(fa, w)
    O, LSE = oracle.attention_varlen_ref(bits(w.q), bits(w.k), bits(w.v), w.cu_seqlens,
                                         w.cu_seqlens, w.scale, causal, window)
    check(f"varlen run{case}", o, lse, O, LSE)
    # the same tiles run the same code: identical bits to the unplanned call
    cu = dev(torch.from_numpy(w.cu_seqlens))
    o2, lse2 = fa.fa_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), cu, cu, w.max_seqlen,
                                w.max_seqlen, w.scale, causal, window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.cpu().view(torch.int16))
    assert torch.equal(lse, lse2.cpu())


def test_varlen_run_any_order_and_partial_plans(fa):
    w = workloads.random_varlen(911, [300, 5, 0, 200, 129], 4, 2, 128, True, (100, 0))
    plan = fa.fa_varlen_plan(w.cu_seqlens, w.cu_seqlens, w.causal, w.window)
    ref_o, ref_l = run_planned(fa, w, plan)
    rng = np.random.default_rng(7)
    o, l = run_planned(fa, w, plan[rng.permutation(len(plan))])
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)) and torch.equal(l, ref_l)
    # a partial plan with items that name no tile: listed tiles are computed,
    # unlisted rows keep the caller's values, bad items are skipped
    keep = plan[::2]
    bad = np.array([[5, 0], [-1, 0], [0, 3], [1, -1], [3, 2]], dtype=np.int32)
    part = np.concatenate([keep, bad])
    sent_o = torch.full_like(w.q, 7.0, device="cuda")
    sent_l = torch.full((w.q.shape[1], w.q.shape[0]), 7.0, dtype=torch.float32, device="cuda")
    o, l = run_planned(fa, w, part, out=sent_o, lse=sent_l)
    listed = np.zeros(w.q.shape[0], dtype=bool)
    for b, t in keep.tolist():
        s0 = int(w.cu_seqlens[b]) + 128 * t
        listed[s0:min(s0 + 128, int(w.cu_seqlens[b + 1]))] = True
    idx = torch.from_numpy(listed)
    assert torch.equal(o[idx].view(torch.int16), ref_o[idx].view(torch.int16))
    assert torch.equal(l[:, idx], ref_l[:, idx])
    assert (o[~idx] == 7.0).all() and (l[:, ~idx] == 7.0).all()


# ---------------------------------------------------------- full workloads
# The named workloads at full size, in the launch configuration bench.py times.
# Outputs start NaN-poisoned, so an element no workgroup writes fails, and
# every output element is compared with the oracle (row blocks of at most 1024
# query rows, run in a thread pool on the host).
def rows_in_blocks(rows, block=1024):
    rows = np.asarray(rows)
    return [rows[i:i + block] for i in range(0, len(rows), block)]


def run_dense_poisoned(fa, w):
    q = dev(w.q)
    B, Lq, Hq, _ = w.q.shape
    out = nan_like(q)
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device="cuda")
    o, l = fa.fa_fwd(q, dev(w.k), dev(w.v), w.scale, w.causal, w.window, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
    return f64(o.cpu()), f64(l.cpu())


def check_dense_tasks(name, w, o_np, lse_np, tasks):
    """Every output finite, then each (b, h, rows) task against the oracle."""
    assert np.isfinite(o_np).all(), f"{name}: non-finite (unwritten?) output"
    assert np.isfinite(lse_np).all(), f"{name}: non-finite (unwritten?) LSE"
    qb, kb, vb = bits(w.q), bits(w.k), bits(w.v)
    refs = oracle_rows_parallel(qb, kb, vb, tasks, w.scale, w.causal, w.window)
    worst = (0.0, 0.0)
    for (b, h, rows), (O, LSE) in zip(tasks, refs):
        r = check(f"{name} b{b} h{h} rows {rows[0]}..{rows[-1]} ({len(rows)})",
                  o_np[b, rows, h], lse_np[b, h, rows], O, LSE)
        worst = (max(worst[0], r[0]), max(worst[1], r[1]))
    print(f"[parity] {name}: {len(tasks)} row blocks, worst err/tol {worst[0]:.3f}, "
          f"worst |dLSE| {worst[1]:.2e}", flush=True)
    return worst


def test_full_causal_mha(fa):
    w = workloads.causal_mha()
    o, lse = run_dense_poisoned(fa, w)
    B, L, H, _ = w.q.shape
    tasks = [(b, h, rows) for b in range(B) for h in range(H) for rows in rows_in_blocks(np.arange(L))]
    check_dense_tasks(w.name, w, o, lse, tasks)


def test_full_causal_gqa_long(fa):
    w = workloads.causal_gqa_long()
    o, lse = run_dense_poisoned(fa, w)
    _, L, H, _ = w.q.shape
    tasks = [(0, h, rows) for h in range(H) for rows in rows_in_blocks(np.arange(L))]
    check_dense_tasks(w.name, w, o, lse, tasks)


@pytest.mark.parametrize("planned", [False, True], ids=["all_split_slots", "planned"])
def test_full_paged_decode(fa, planned):
    w = workloads.paged_decode()
    o, lse = run_decode_planned(fa, w) if planned else run_decode(fa, w)
    O, LSE = decode_ref(w)
    check(w.name, o, lse, O, LSE)


@pytest.mark.parametrize("planned", [False, True], ids=["sequence_order", "planned"])
def test_full_varlen_window(fa, planned):
    w = workloads.varlen_window()
    cu = dev(torch.from_numpy(w.cu_seqlens))
    q = dev(w.q)
    T, H, _ = w.q.shape
    out = nan_like(q)
    lse_buf = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    if planned:
        o, lse = run_planned(fa, w, out=out, lse=lse_buf)
    else:
        o, lse = fa.fa_fwd_varlen(q, dev(w.k), dev(w.v), cu, cu, w.max_seqlen,
                                  w.max_seqlen, w.scale, w.causal, w.window, out=out, lse=lse_buf)
        torch.cuda.synchronize()
    o, lse = f64(o.cpu()), f64(lse.cpu())
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "unwritten varlen output"
    # each packed sequence is the dense definition on its own slice (a batch of one)
    qb, kb, vb = bits(w.q), bits(w.k), bits(w.v)
    worst = (0.0, 0.0)
    for b, L in enumerate(w.lens):
        s, L = int(w.cu_seqlens[b]), int(L)
        sub = [(0, h, rows) for h in range(H) for rows in rows_in_blocks(np.arange(L))]
        refs = oracle_rows_parallel(qb[None, s:s + L], kb[None, s:s + L], vb[None, s:s + L], sub,
                                    w.scale, w.causal, w.window)
        for (_, h, rows), (O, LSE) in zip(sub, refs):
            r = check(f"{w.name} seq{b} h{h} rows {rows[0]}..{rows[-1]}", o[s + rows, h],
                      lse[h, s + rows], O, LSE)
            worst = (max(worst[0], r[0]), max(worst[1], r[1]))
    print(f"[parity] {w.name}: every element, worst err/tol {worst[0]:.3f}, "
          f"worst |dLSE| {worst[1]:.2e}", flush=True)


# ------------------------------------------- chunked prefill over a paged cache
def run_kvcache(fa, w):
    """fa_fwd_kvcache on device copies; returns O, LSE and the caches after it."""
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    kn = dev(w.k_new) if w.k_new is not None else None
    vn = dev(w.v_new) if w.v_new is not None else None
    o, lse = fa.fa_fwd_kvcache(dev(w.q), kc, vc, dev(torch.from_numpy(w.block_table)),
                               dev(torch.from_numpy(w.cache_seqlens)), kn, vn, w.scale, w.causal,
                               w.window)
    torch.cuda.synchronize()
    return o, lse, kc.cpu(), vc.cpu()


def kvcache_ref(w):
    kn = bits(w.k_new) if w.k_new is not None else None
    vn = bits(w.v_new) if w.v_new is not None else None
    return oracle.attention_kvcache_ref(bits(w.q), bits(w.k_cache), bits(w.v_cache), w.block_table,
                                        w.cache_seqlens, w.page_size, kn, vn, w.scale, w.causal,
                                        w.window)


# (cached lengths, Lq, Hq, Hkv, d, page_size, append, causal, window)
KVCACHE_CASES = [
    ([300, 17, 1000], 70, 8, 2, 128, 16, True, True, (-1, -1)),
    ([0, 129, 64], 130, 4, 4, 64, 16, True, True, (-1, -1)),      # an empty cache
    ([513, 200], 1, 8, 1, 128, 32, False, True, (-1, -1)),        # one query row, no append
    ([1000, 300], 257, 8, 2, 128, 16, False, True, (100, 0)),     # keys fewer than queries
    ([77, 400], 33, 6, 3, 64, 48, True, False, (-1, -1)),         # non-causal, 48-token pages
    ([2000, 5], 300, 8, 8, 128, 16, True, True, (64, 0)),         # window across the append
    ([0, 0], 5, 2, 1, 128, 16, False, True, (-1, -1)),            # nothing to attend to
]


@pytest.mark.parametrize("case", KVCACHE_CASES,
                         ids=lambda c: f"n{len(c[0])}-lq{c[1]}-h{c[2]}-kv{c[3]}-d{c[4]}-p{c[5]}-a{int(c[6])}-c{int(c[7])}-w{c[8][0]}")
def test_kvcache_sweep(fa, case):
    lens, Lq, Hq, Hkv, d, ps, append, causal, window = case
    w = workloads.random_kvcache(600 + sum(lens) + Lq, lens, Lq, Hq, Hkv, d, ps, append, causal, window)
    o, lse, kc, vc = run_kvcache(fa, w)
    O, LSE, kc_ref, vc_ref = kvcache_ref(w)
    check(f"kvcache{case}", o, lse, O, LSE)
    # the append wrote exactly the new rows, bit for bit, and nothing else
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)


def test_full_chunked_prefill(fa):
    w = workloads.chunked_prefill()
    o, lse, kc, vc = run_kvcache(fa, w)
    O, LSE, kc_ref, vc_ref = kvcache_ref(w)
    check(w.name, o, lse, O, LSE)
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)


# ------------------------------------------------- softcap and ALiBi modifiers
def alibi_slopes(Hq, B=None):
    """The usual geometric ALiBi slopes 2^(-8 (h + 1) / Hq); per batch, scaled
    by (b + 1) / B so each request differs."""
    base = np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)])
    if B is None:
        return base.astype(np.float32)
    return np.stack([base * (b + 1) / B for b in range(B)]).astype(np.float32)


# B, Lq, Lk, Hq, Hkv, d, causal, window, softcap, alibi ("none" | "head" | "batch")
MOD_CASES = [
    (2, 300, 300, 4, 2, 128, True, (-1, -1), 30.0, "none"),
    (2, 300, 300, 4, 2, 128, True, (-1, -1), 0.0, "head"),
    (2, 257, 257, 8, 2, 128, True, (64, 0), 5.0, "batch"),
    (1, 129, 385, 4, 1, 64, True, (-1, -1), 2.0, "head"),
    (1, 200, 200, 2, 2, 64, False, (-1, -1), 0.5, "batch"),
]


@pytest.mark.parametrize("case", MOD_CASES, ids=lambda c: f"L{c[1]}x{c[2]}-h{c[3]}-d{c[5]}-c{int(c[6])}-cap{c[8]}-{c[9]}")
def test_dense_score_modifiers(fa, case):
    B, Lq, Lk, Hq, Hkv, d, causal, window, cap, al = case
    w = workloads.random_dense(700 + Lq + Lk + Hq, B, Lq, Lk, Hq, Hkv, d, causal, window)
    slopes = None if al == "none" else alibi_slopes(Hq, B if al == "batch" else None)
    o, lse = fa.fa_fwd(dev(w.q), dev(w.k), dev(w.v), w.scale, causal, window, softcap=cap,
                       alibi_slopes=None if slopes is None else dev(torch.from_numpy(slopes)))
    torch.cuda.synchronize()
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), w.scale, causal, window,
                                  softcap=cap, alibi_slopes=slopes)
    check(f"mods{case}", o, lse, O, LSE)


def test_varlen_and_kvcache_score_modifiers(fa):
    w = workloads.random_varlen(731, [70, 300, 5, 160], 8, 2, 128, True, (-1, -1))
    slopes = alibi_slopes(8, 4)
    cu = dev(torch.from_numpy(w.cu_seqlens))
    o, lse = fa.fa_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), cu, cu, w.max_seqlen, w.max_seqlen,
                              w.scale, True, (-1, -1), softcap=8.0,
                              alibi_slopes=dev(torch.from_numpy(slopes)))
    torch.cuda.synchronize()
    O, LSE = oracle.attention_varlen_ref(bits(w.q), bits(w.k), bits(w.v), w.cu_seqlens, w.cu_seqlens,
                                         w.scale, True, (-1, -1), softcap=8.0, alibi_slopes=slopes)
    check("varlen mods", o, lse, O, LSE)

    kv = workloads.random_kvcache(732, [300, 17], 70, 8, 2, 128, 16, True, True)
    sl = alibi_slopes(8)
    kc, vc = dev(kv.k_cache), dev(kv.v_cache)
    o, lse = fa.fa_fwd_kvcache(dev(kv.q), kc, vc, dev(torch.from_numpy(kv.block_table)),
                               dev(torch.from_numpy(kv.cache_seqlens)), dev(kv.k_new), dev(kv.v_new),
                               kv.scale, True, softcap=20.0, alibi_slopes=dev(torch.from_numpy(sl)))
    torch.cuda.synchronize()
    O, LSE, _, _ = oracle.attention_kvcache_ref(bits(kv.q), bits(kv.k_cache), bits(kv.v_cache),
                                                kv.block_table, kv.cache_seqlens, kv.page_size,
                                                bits(kv.k_new), bits(kv.v_new), kv.scale, True,
                                                softcap=20.0, alibi_slopes=sl)
    check("kvcache mods", o, lse, O, LSE)


@pytest.mark.parametrize("case", [
    # lens, Hq, Hkv, d, page_size, split, window_left, softcap, alibi
    ([1000, 17, 513], 32, 8, 128, 16, 512, -1, 0.5, "none"),     # four-head sets
    ([1000, 17, 513], 32, 8, 128, 16, 256, 300, 0.0, "head"),
    ([700, 33, 129], 16, 2, 128, 32, 64, -1, 1.0, "batch"),      # two-head sets (8 per KV head)
    ([700, 33, 129], 48, 4, 64, 16, 512, 100, 2.0, "head"),      # 12 per KV head, d = 64
    ([300, 7, 900], 8, 2, 128, 8, 128, -1, 0.7, "batch"),        # general kernel (page size 8)
    ([300, 7, 900], 16, 1, 64, 16, 128, 200, 0.0, "batch"),      # general kernel, one KV head
])
def test_decode_score_modifiers(fa, case):
    """softcap and ALiBi in paged decode, unplanned and planned (the query at
    position len - 1)."""
    lens, Hq, Hkv, d, ps, split, wl, cap, al = case
    npages = sum(-(-l // ps) for l in lens) + 3
    w = workloads.random_paged(900 + Hq + d + ps, lens, Hq, Hkv, d, ps, npages, split,
                               window_left=wl)
    slopes = None if al == "none" else alibi_slopes(Hq, len(lens) if al == "batch" else None)
    sl_dev = None if slopes is None else dev(torch.from_numpy(slopes))
    O, LSE = oracle.decode_paged_ref(bits(w.q), bits(w.k_cache), bits(w.v_cache), w.block_table,
                                     w.seqlens, w.page_size, w.scale, wl, softcap=cap,
                                     alibi_slopes=slopes)
    args = (dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(torch.from_numpy(w.block_table)),
            dev(torch.from_numpy(w.seqlens)))
    o, lse = fa.fa_decode_paged(*args, w.scale, wl, split, softcap=cap, alibi_slopes=sl_dev)
    torch.cuda.synchronize()
    check(f"decode mods{case}", o.cpu(), lse.cpu(), O, LSE)
    plan = fa.fa_decode_plan(w.seqlens, ps, w.block_table.shape[1], wl, split)
    o2, lse2 = fa.fa_decode_paged_run(*args, dev(torch.from_numpy(np.ascontiguousarray(plan))),
                                      w.scale, wl, split, softcap=cap, alibi_slopes=sl_dev)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("Hq,Hkv,d", [(16, 4, 128), (8, 2, 64)])
def test_decode_many_requests(fa, Hq, Hkv, d):
    """More requests than the device-made work order takes per pass (1024):
    lengths 0..90 with 16-token splits and a window mix empty requests, full
    and partial splits; unplanned and planned results agree bit for bit."""
    rng = np.random.default_rng(950 + Hq + d)
    lens = [int(x) for x in rng.integers(0, 91, 2100)]
    ps, split, wl = 16, 16, 40
    npages = sum(-(-l // ps) for l in lens) + 3
    w = workloads.random_paged(951 + d, lens, Hq, Hkv, d, ps, npages, split,
                               max_blocks=6, window_left=wl)
    o, lse = run_decode(fa, w)
    O, LSE = decode_ref(w)
    check(f"decode many requests h{Hq} kv{Hkv} d{d}", o, lse, O, LSE)
    o2, lse2 = run_decode_planned(fa, w)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("B,Hq,Hkv,wl", [(200, 32, 8, 700), (256, 64, 8, -1), (65, 16, 4, 300)])
def test_decode_self_ordered_batches(fa, B, Hq, Hkv, wl):
    """Unplanned head-set launches of up to 256 requests find their own work
    items (several 64-request passes): lengths from 0 to 3000 with 256-token
    splits, with and without a window, so full, partial-first, partial-last and
    empty requests mix; the result agrees with the oracle, and bit for bit
    with the planned run over the same cache."""
    rng = np.random.default_rng(4000 + B + Hq)
    lens = [int(x) for x in rng.integers(0, 3001, B)]
    lens[0], lens[-1] = 0, 512
    ps, split = 16, 256
    npages = sum(-(-l // ps) for l in lens) + 3
    w = workloads.random_paged(4100 + B, lens, Hq, Hkv, 128, ps, npages, split,
                               max_blocks=190, window_left=wl)
    o, lse = run_decode(fa, w)
    O, LSE = decode_ref(w)
    check(f"decode self-ordered B{B} h{Hq} kv{Hkv} w{wl}", o, lse, O, LSE)
    o2, lse2 = run_decode_planned(fa, w)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


# ------------------------------------------------ wide-tile kernel (d = 128)
# fa_fwd takes the 256-row wide-tile kernel for head_dim 128 from 4096 query
# rows on; these cases sit just past that, with ragged row and 64-key tails,
# so every mask mode, GQA (workgroups of 1, 2 and 4 query heads), Lq != Lk,
# the rescale paths and the score modifiers run through it (the smaller dense
# cases above take the narrow one).
WIDE_CASES = [
    # B, Lq, Lk, Hq, Hkv, causal, window, softcap, alibi
    (1, 4133, 4133, 2, 1, True, (-1, -1), 0.0, "none"),
    (1, 4096, 4096, 2, 2, False, (-1, -1), 0.0, "none"),
    (1, 4100, 4500, 2, 1, True, (-1, -1), 0.0, "none"),     # Lq < Lk: bottom-right causal
    (1, 4500, 4100, 2, 2, True, (-1, -1), 0.0, "none"),     # Lq > Lk: first 400 rows see no key
    (1, 4111, 4111, 4, 2, True, (300, 0), 0.0, "none"),     # sliding window
    (1, 4099, 4099, 2, 1, False, (200, 37), 0.0, "none"),   # two-sided window
    (2, 4097, 4097, 2, 1, True, (-1, -1), 20.0, "head"),    # softcap + ALiBi
    (1, 4160, 4160, 2, 2, True, (64, 0), 0.0, "batch"),
    # 4 query heads per KV head: 64-row workgroups of 4 heads ("head sets")
    (1, 4133, 4133, 4, 1, True, (-1, -1), 0.0, "none"),
    (1, 4500, 4100, 8, 2, True, (-1, -1), 0.0, "none"),     # Lq > Lk, two KV groups
    (1, 4111, 4111, 8, 1, True, (300, 0), 20.0, "head"),    # two head sets per KV group
    # 6 query heads per KV head: 2-head workgroups of 128 rows
    (1, 4100, 4500, 6, 1, False, (200, 37), 0.0, "none"),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: f"L{c[1]}x{c[2]}-h{c[3]}_{c[4]}-c{int(c[5])}-w{c[6][0]}_{c[6][1]}-cap{c[7]}-{c[8]}")
def test_wide_kernel_sweep(fa, case):
    B, Lq, Lk, Hq, Hkv, causal, window, cap, al = case
    w = workloads.random_dense(900 + Lq + Lk + Hq, B, Lq, Lk, Hq, Hkv, 128, causal, window)
    slopes = None if al == "none" else alibi_slopes(Hq, B if al == "batch" else None)
    q = dev(w.q)
    out = nan_like(q)
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device="cuda")
    o, l = fa.fa_fwd(q, dev(w.k), dev(w.v), w.scale, causal, window, out=out, lse=lse, softcap=cap,
                     alibi_slopes=None if slopes is None else dev(torch.from_numpy(slopes)))
    torch.cuda.synchronize()
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), w.scale, causal, window,
                                  softcap=cap, alibi_slopes=slopes)
    check(f"wide{case}", o.cpu(), l.cpu(), O, LSE)


@pytest.mark.parametrize("kind", ["rising", "large_scale"])
def test_wide_kernel_rescale_paths(fa, kind):
    """Scores that rise along the keys (the max is raised on many tiles, through
    both the up-front and the after-the-block paths), and a large scale that
    makes P nearly one-hot, through the wide-tile kernel."""
    B, L, H = 1, 4200, 2
    if kind == "rising":
        w = workloads.random_dense(77, B, L, L, H, H, 128, True)
        k = w.k.float()
        qdir = w.q.float()[:, -1:, :, :] / w.q.float()[:, -1:, :, :].norm(dim=-1, keepdim=True)
        w.k = (k + torch.linspace(0, 40, L).view(1, L, 1, 1) * qdir).to(torch.bfloat16)
        scale = w.scale
    else:
        w = workloads.random_dense(78, B, L, L, H, 1, 128, True, scale=2.0)
        scale = 2.0
    o, lse = run_dense(fa, w)
    O, LSE = oracle.attention_ref(bits(w.q), bits(w.k), bits(w.v), scale, True)
    check(f"wide_{kind}", o, lse, O, LSE)
