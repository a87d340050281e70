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
