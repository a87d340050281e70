"""The -DFA_DEBUG build (libfa_debug.so) fills the LDS destination of every
direct-to-LDS tile load with bf16 NaN before the load.  A read that a missing
wait or barrier let through would then return NaN, and NaN reaches the
outputs; with correct synchronisation no poisoned byte is ever read, so the
debug build must agree bit for bit with the release build on every kernel that
stages tiles through LDS (narrow and wide prefill, chunked prefill over a paged
cache, the backward kernels)."""

import ctypes
import os

import numpy as np
import pytest
import torch

import exact_attention_17_amd as fa_mod
import workloads
from exact_attention_17_amd import build
from gpu_helpers import dev


def test_debug_library_exports_every_symbol():
    if not os.path.exists(build.DEBUG_LIB_PATH):
        build.build_library(debug=True)
    lib = ctypes.CDLL(build.DEBUG_LIB_PATH)
    for name in fa_mod.exported_symbols():
        assert hasattr(lib, name), name


@pytest.fixture(scope="module")
def debug_lib(fa):
    if not os.path.exists(build.DEBUG_LIB_PATH):
        pytest.fail("libfa_debug.so is missing: build it with `python -m exact_attention_17_amd.build`")
    release = fa_mod.load_library()
    dbg = fa_mod.load_library(build.DEBUG_LIB_PATH)     # loads a second handle ...
    fa_mod._lib = release                                # ... and leaves the release one current
    return release, dbg


def _both(libs, call):
    """call() under the release library and under the debug one."""
    out = []
    for lib in libs:
        saved = fa_mod._lib
        fa_mod._lib = lib
        try:
            r = call()
            torch.cuda.synchronize()
            out.append([t.clone() for t in r])
        finally:
            fa_mod._lib = saved
    return out


def _same(a, b):
    for x, y in zip(a, b):
        xv = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
        yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
        assert torch.equal(xv, yv)


DENSE = [
    # B, Lq, Lk, Hq, Hkv, d, causal, window
    (2, 333, 333, 8, 2, 128, True, (-1, -1)),       # narrow, d = 128
    (1, 700, 900, 4, 4, 64, True, (100, 0)),        # narrow, d = 64, window
    (1, 4133, 4133, 8, 2, 128, True, (-1, -1)),     # wide, 4-head workgroups
    (1, 4500, 4100, 2, 2, 128, False, (300, 40)),   # wide, 1-head workgroups
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", DENSE)
def test_debug_build_matches_release_dense(debug_lib, case):
    B, Lq, Lk, Hq, Hkv, d, causal, window = case
    w = workloads.random_dense(880 + Lq + d, B, Lq, Lk, Hq, Hkv, d, causal, window)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    a, b = _both(debug_lib, lambda: fa_mod.fa_fwd(q, k, v, w.scale, causal, window))
    _same(a, b)
    assert torch.isfinite(a[0].float()).all()


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
def test_debug_build_matches_release_varlen_and_backward(debug_lib, d):
    w = workloads.random_varlen(890 + d, [5, 300, 1, 129, 700], 4, 2, d, True, (-1, -1))
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    cu = dev(torch.from_numpy(w.cu_seqlens))
    mx = int(np.diff(w.cu_seqlens).max())
    a, b = _both(debug_lib, lambda: fa_mod.fa_fwd_varlen(q, k, v, cu, cu, mx, mx, w.scale, True))
    _same(a, b)
    wd = workloads.random_dense(895 + d, 2, 300, 300, 4, 2, d, True)
    qd, kd, vd = dev(wd.q), dev(wd.k), dev(wd.v)
    do = dev(workloads.upstream_grad(896 + d, tuple(wd.q.shape)))
    o, lse = fa_mod.fa_fwd(qd, kd, vd, wd.scale, True)
    torch.cuda.synchronize()
    a, b = _both(debug_lib, lambda: fa_mod.fa_bwd(qd, kd, vd, o, lse, do, wd.scale, True))
    _same(a, b)


@pytest.mark.gpu
def test_debug_build_matches_release_chunked_prefill(debug_lib):
    w = workloads.random_kvcache(897, [300, 17, 650], 64, 8, 2, 128, 16, True, True)
    def call():
        kc, vc = dev(w.k_cache), dev(w.v_cache)
        o, lse = fa_mod.fa_fwd_kvcache(dev(w.q), kc, vc, dev(torch.from_numpy(w.block_table)),
                                       dev(torch.from_numpy(w.cache_seqlens)), dev(w.k_new),
                                       dev(w.v_new), w.scale, w.causal, w.window)
        return o, lse, kc, vc
    a, b = _both(debug_lib, call)
    _same(a, b)


# ---- device-side preconditions (debug build only) ---------------------------
# Each bad input below goes to the debug library alone, which must reject it
# with FA_ERR_INVALID_ARG before any other kernel runs.  The inputs are laid
# out so that even an unchecked read would stay inside mapped memory: the
# page pool passed in is a slice of a larger one (page ids -1 and num_pages
# exist), and over-long requests sit in row 0 of the block table.

def _expect_invalid(libs, call):
    saved = fa_mod._lib
    fa_mod._lib = libs[1]
    try:
        with pytest.raises(fa_mod.FAError) as err:
            call()
        torch.cuda.synchronize()
    finally:
        fa_mod._lib = saved
    assert err.value.status == 1


def _paged_case():
    p = workloads.random_paged(901, [300, 17, 650], 8, 2, 128, 16, 80, 256, max_blocks=48)
    big_k = torch.cat([p.k_cache[:1], p.k_cache, p.k_cache[:1]]).cuda()
    big_v = torch.cat([p.v_cache[:1], p.v_cache, p.v_cache[:1]]).cuda()
    n = p.k_cache.shape[0]
    return p, big_k[1:n + 1], big_v[1:n + 1], n


@pytest.mark.gpu
def test_debug_build_rejects_bad_page_ids_and_lengths(debug_lib):
    p, kc, vc, n = _paged_case()
    q = dev(p.q)
    lens = dev(torch.as_tensor(p.seqlens))

    def decode(table, sl):
        return fa_mod.fa_decode_paged(q, kc, vc, dev(torch.as_tensor(table)), sl, p.scale, -1, 256)

    # a valid call, and one with out-of-range ids only in entries past each
    # request's pages (allowed), agree with the release library bit for bit
    a, b = _both(debug_lib, lambda: decode(p.block_table, lens))
    _same(a, b)
    loose = p.block_table.copy()
    for r, L in enumerate(p.seqlens):
        loose[r, -(-int(L) // 16):] = 10 ** 6
    a, b = _both(debug_lib, lambda: decode(loose, lens))
    _same(a, b)
    for bad_id in (-1, n):
        t = p.block_table.copy()
        t[0, 3] = bad_id
        _expect_invalid(debug_lib, lambda: decode(t, lens))
    long_lens = torch.as_tensor(p.seqlens).clone()
    long_lens[0] = 48 * 16 + 1
    _expect_invalid(debug_lib, lambda: decode(p.block_table, dev(long_lens)))
    neg = torch.as_tensor(p.seqlens).clone()
    neg[0] = -1
    _expect_invalid(debug_lib, lambda: decode(p.block_table, dev(neg)))


@pytest.mark.gpu
def test_debug_build_rejects_bad_kvcache_before_appending(debug_lib):
    w = workloads.random_kvcache(902, [300, 17], 64, 8, 2, 128, 16, True, True)
    pool = w.k_cache.shape[0]
    spare = torch.zeros((8,) + tuple(w.k_cache.shape[1:]), dtype=torch.bfloat16)
    kc = torch.cat([w.k_cache, spare]).cuda()[:pool]
    vc = torch.cat([w.v_cache, spare]).cuda()[:pool]
    k0, v0 = kc.clone(), vc.clone()
    table = w.block_table.copy()
    table[0, 0] = pool + 5
    sl = dev(torch.from_numpy(w.cache_seqlens))

    def call(t, lens):
        return fa_mod.fa_fwd_kvcache(dev(w.q), kc, vc, dev(torch.from_numpy(t)), lens, dev(w.k_new),
                                     dev(w.v_new), w.scale, True)

    _expect_invalid(debug_lib, lambda: call(table, sl))
    # row 0 would need one token more than its table holds once the chunk is appended
    over = torch.from_numpy(w.cache_seqlens.copy())
    over[0] = w.block_table.shape[1] * 16 - 64 + 1
    _expect_invalid(debug_lib, lambda: call(w.block_table, dev(over)))
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), v0.view(torch.int16))


@pytest.mark.gpu
def test_debug_build_rejects_bad_cu_seqlens(debug_lib):
    w = workloads.random_varlen(903, [100, 200, 150], 4, 2, 64, True)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    good = w.cu_seqlens

    def fwd(cu, mx=200):
        c = dev(torch.from_numpy(np.asarray(cu, dtype=np.int32)))
        return fa_mod.fa_fwd_varlen(q, k, v, c, c, mx, mx, w.scale, True)

    a, b = _both(debug_lib, lambda: fwd(good))
    _same(a, b)
    for cu, mx in (([5, 100, 300, 450], 200),      # does not start at 0
                   ([0, 200, 100, 450], 350),      # decreasing
                   ([0, 100, 300, 440], 200),      # does not end at total
                   ([0, 100, 300, 450], 150)):     # a sequence longer than max_seqlen
        _expect_invalid(debug_lib, lambda: fwd(cu, mx))
    o, lse = fwd(good)
    do = dev(workloads.upstream_grad(904, tuple(w.q.shape)))
    torch.cuda.synchronize()
    short = dev(torch.from_numpy(np.asarray([0, 100, 300, 440], dtype=np.int32)))
    _expect_invalid(debug_lib, lambda: fa_mod.fa_bwd_varlen(q, k, v, o, lse, do, short, short, 200,
                                                            200, w.scale, True))
