"""GPU properties of the HIP path that hold at any size (no oracle needed for
the bitwise ones): run-to-run determinism, invariance to page-id permutation
and to the contents of unused pages, GQA == MHA with repeated KV heads,
varlen == per-sequence dense calls, split-size invariance, and decode ==
the last row of causal prefill over the same keys."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bits, check, dev, f64

pytestmark = pytest.mark.gpu


def decode(fa, q, kc, vc, table, lens, scale, split=0, window_left=-1):
    o, lse = fa.fa_decode_paged(dev(q), dev(kc), dev(vc), dev(torch.as_tensor(table)),
                                dev(torch.as_tensor(lens)), scale, window_left, split)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def test_bitwise_determinism(fa):
    w = workloads.random_dense(11, 2, 700, 700, 8, 2, 128, True, (300, 0))
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    a = fa.fa_fwd(q, k, v, w.scale, True, (300, 0))
    b = fa.fa_fwd(q, k, v, w.scale, True, (300, 0))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    p = workloads.random_paged(12, [900, 33, 1500], 8, 2, 128, 16, 200, 256)
    r1 = decode(fa, p.q, p.k_cache, p.v_cache, p.block_table, p.seqlens, p.scale, 256)
    r2 = decode(fa, p.q, p.k_cache, p.v_cache, p.block_table, p.seqlens, p.scale, 256)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_page_permutation_and_unused_pages(fa):
    p = workloads.random_paged(13, [1000, 17, 640], 8, 2, 128, 16, 160, 512)
    base = decode(fa, p.q, p.k_cache, p.v_cache, p.block_table, p.seqlens, p.scale)
    rng = np.random.default_rng(13)
    perm = rng.permutation(p.k_cache.shape[0])
    inv = np.argsort(perm)
    kc, vc = p.k_cache[torch.from_numpy(perm)], p.v_cache[torch.from_numpy(perm)]
    table = inv[p.block_table].astype(np.int32)
    moved = decode(fa, p.q, kc, vc, table, p.seqlens, p.scale)
    assert torch.equal(base[0], moved[0]) and torch.equal(base[1], moved[1])
    # garbage (huge values and inf) in unused pages and tail slots changes nothing
    used = np.zeros(p.k_cache.shape[0], bool)
    for b, L in enumerate(p.seqlens):
        used[p.block_table[b, :-(-int(L) // 16)]] = True
    kc2, vc2 = p.k_cache.clone(), p.v_cache.clone()
    kc2[torch.from_numpy(~used)] = 3.0e38
    vc2[torch.from_numpy(~used)] = float("-inf")
    nan_slots = torch.isnan(kc2.float())
    kc2[nan_slots] = float("inf")
    vc2[torch.isnan(vc2.float())] = 1.0e30
    dirty = decode(fa, p.q, kc2, vc2, p.block_table, p.seqlens, p.scale)
    assert torch.equal(base[0], dirty[0]) and torch.equal(base[1], dirty[1])


def test_gqa_equals_repeated_mha(fa):
    w = workloads.random_dense(14, 2, 333, 333, 8, 2, 128, True)
    a = fa.fa_fwd(dev(w.q), dev(w.k), dev(w.v), w.scale, True)
    kr = w.k.repeat_interleave(4, dim=2).contiguous()
    vr = w.v.repeat_interleave(4, dim=2).contiguous()
    b = fa.fa_fwd(dev(w.q), dev(kr), dev(vr), w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_equals_per_sequence_dense(fa):
    lens = [200, 1, 129, 64, 450]
    w = workloads.random_varlen(15, lens, 4, 2, 64, True, (100, 0))
    cu = dev(torch.from_numpy(w.cu_seqlens))
    o, lse = fa.fa_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), cu, cu, w.max_seqlen, w.max_seqlen,
                              w.scale, True, (100, 0))
    for b, L in enumerate(lens):
        s = int(w.cu_seqlens[b])
        od, lsed = fa.fa_fwd(dev(w.q[None, s:s + L]), dev(w.k[None, s:s + L]), dev(w.v[None, s:s + L]),
                             w.scale, True, (100, 0))
        assert torch.equal(o[s:s + L], od[0]), b
        assert torch.equal(lse[:, s:s + L], lsed[0]), b


@pytest.mark.parametrize("split", [16, 64, 512, 8192])
def test_split_size_invariance(fa, split):
    p = workloads.random_paged(16, [2000, 700, 31], 8, 2, 128, 16, 200, split)
    o, lse = decode(fa, p.q, p.k_cache, p.v_cache, p.block_table, p.seqlens, p.scale, split)
    O, LSE = oracle.decode_paged_ref(bits(p.q), bits(p.k_cache), bits(p.v_cache), p.block_table,
                                     p.seqlens, 16, p.scale)
    check(f"split{split}", o, lse, O, LSE)


def test_decode_equals_last_prefill_row(fa):
    L, Hq, Hkv, d = 777, 8, 2, 128
    w = workloads.random_dense(17, 1, L, L, Hq, Hkv, d, True)
    o_pre, lse_pre = fa.fa_fwd(dev(w.q), dev(w.k), dev(w.v), w.scale, True)
    # scatter the same K/V into 16-token pages in reversed page order
    npg = -(-L // 16)
    kc = torch.zeros(npg + 1, 16, Hkv, d, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    table = np.zeros((1, npg), np.int32)
    for j in range(npg):
        pid = npg - j
        table[0, j] = pid
        n = min(16, L - 16 * j)
        kc[pid, :n] = w.k[0, 16 * j:16 * j + n]
        vc[pid, :n] = w.v[0, 16 * j:16 * j + n]
    o_dec, lse_dec = decode(fa, w.q[:, -1:], kc, vc, table, np.array([L], np.int32), w.scale, 128)
    O, LSE = oracle.attention_rows_ref(bits(w.q), bits(w.k), bits(w.v), 0, 0, [L - 1], w.scale, True)
    a, b = f64(o_dec)[0, 0], f64(o_pre.cpu())[0, -1]
    assert np.abs(a - b).max() <= 2 * (4e-3 + 1e-2 * np.abs(b).max())
    assert abs(float(lse_dec[0, 0]) - float(lse_pre.cpu()[0, 0, -1])) <= 2e-4
    check("decode_vs_oracle_row", o_dec[0, 0, :1].float(), lse_dec[0, :1], O, LSE)


def test_repeated_runs_are_bitwise_identical(fa):
    """Many short workgroups, run repeatedly: an LDS reuse race between waves
    would show up as run-to-run differences."""
    for case in [(1, 160, 160, 4, 2, 64, False, (-1, -1)), (2, 300, 300, 4, 2, 128, True, (-1, -1))]:
        B, Lq, Lk, Hq, Hkv, d, causal, window = case
        w = workloads.random_dense(31, B, Lq, Lk, Hq, Hkv, d, causal, window)
        q, k, v = dev(w.q), dev(w.k), dev(w.v)
        ref = fa.fa_fwd(q, k, v, w.scale, causal, window)
        for _ in range(30):
            o, lse = fa.fa_fwd(q, k, v, w.scale, causal, window)
            assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), case


def test_side_stream_calls_match_current_stream_calls(fa):
    """Calls on a side stream (buffers the binding allocates live on that stream)
    return bitwise what calls on the current stream return; the side stream's
    results are read after it is synchronised, while the current stream keeps
    allocating and writing other tensors."""
    w = workloads.random_dense(15, 2, 300, 300, 8, 2, 128, True)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    p = workloads.random_paged(16, [700, 90, 1300], 8, 2, 128, 16, 160, 512)
    pq, kc, vc = dev(p.q), dev(p.k_cache), dev(p.v_cache)
    bt, sl = dev(torch.as_tensor(p.block_table)), dev(torch.as_tensor(p.seqlens))
    do = dev(workloads.upstream_grad(17, tuple(w.q.shape)))
    ref_f = fa.fa_fwd(q, k, v, w.scale, True)
    ref_d = fa.fa_decode_paged(pq, kc, vc, bt, sl, p.scale, -1, 512)
    ref_b = fa.fa_bwd(q, k, v, ref_f[0], ref_f[1], do, w.scale, True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    busy = torch.randn(4096, 4096, device="cuda")
    for _ in range(3):
        with torch.cuda.stream(side):
            for _ in range(4):                  # delay the side stream's kernels, so the
                busy = busy @ busy * 1e-3       # current stream's writes below overlap them
        f = fa.fa_fwd(q, k, v, w.scale, True, stream=side)
        d = fa.fa_decode_paged(pq, kc, vc, bt, sl, p.scale, -1, 512, stream=side)
        g = fa.fa_bwd(q, k, v, ref_f[0], ref_f[1], do, w.scale, True, stream=side)
        junk = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(8)]   # current stream
        side.synchronize()
        for a, b in zip(list(f) + list(d) + list(g), list(ref_f) + list(ref_d) + list(ref_b)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
        del junk


@pytest.mark.parametrize("case", [
    # B, Lq, Lk, Hq, Hkv, causal, window
    (1, 4133, 4133, 8, 2, True, (-1, -1)),      # 4-head workgroups of the wide kernel
    (1, 4500, 4100, 4, 2, True, (-1, -1)),      # 2-head workgroups, Lq > Lk
    (1, 4100, 4600, 2, 2, True, (700, 0)),      # 1-head workgroups, sliding window
    (1, 4096, 3000, 6, 1, False, (300, 20)),    # two-sided window, non-causal
])
def test_wide_and_narrow_kernels_agree_bitwise(fa, case):
    """Dense head_dim-128 prefill from 4096 query rows runs the wide-tile kernel
    (64 rows per wave, up to 4 heads per workgroup); the same problem as a
    one-sequence varlen batch runs the narrow kernel (32 rows per wave).  Both
    take the tiles in the same order with the same per-row arithmetic (base-2
    softmax, the same lazy-rescale decisions per row), so their outputs agree
    bit for bit: a check of each kernel's tiling against the other's."""
    B, Lq, Lk, Hq, Hkv, causal, window = case
    w = workloads.random_dense(60 + Lq + Hq, B, Lq, Lk, Hq, Hkv, 128, causal, window)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o1, l1 = fa.fa_fwd(q, k, v, w.scale, causal, window)
    cu_q = torch.tensor([0, Lq], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, Lk], dtype=torch.int32, device="cuda")
    o2, l2 = fa.fa_fwd_varlen(q[0], k[0], v[0], cu_q, cu_k, Lq, Lk, w.scale, causal, window)
    torch.cuda.synchronize()
    assert torch.equal(o1[0].view(torch.int16), o2.view(torch.int16)), case
    assert torch.equal(l1[0], l2), case
