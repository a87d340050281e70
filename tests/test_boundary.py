"""C-ABI boundary checks that need no GPU: the library loads, exports every
entry point include/fa.h declares, and rejects each invalid argument with its
status code before any HIP call (so nothing is enqueued)."""

import math
import ctypes
import os
import re

import numpy as np
import pytest

import exact_attention_17_amd as fa
from exact_attention_17_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
P = 0x10000          # a fake, 256-byte-aligned "device" address: never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    return fa.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(["fa_status_string", "fa_fwd", "fa_fwd_varlen", "fa_varlen_plan",
                            "fa_fwd_varlen_run", "fa_decode_paged_workspace_size",
                            "fa_decode_paged", "fa_decode_plan", "fa_decode_paged_run",
                            "fa_decode_paged_noalloc",
                            "fa_fwd_kvcache", "fa_bwd", "fa_bwd_workspace_size",
                            "fa_bwd_varlen", "fa_bwd_varlen_workspace_size"])
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(fa.exported_symbols()) == names


def test_status_strings(lib):
    for code in range(5):
        assert lib.fa_status_string(code)
    assert lib.fa_status_string(99) == b"unknown status"


def fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Lq=128, Lk=128, Hq=2, Hkv=1, d=64,
             scale=0.125, causal=0, wl=-1, wr=-1, cap=0.0, al=None, ab=0)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"], a["Lk"], a["Hq"],
                      a["Hkv"], a["d"], a["scale"], a["causal"], a["wl"], a["wr"], a["cap"], a["al"],
                      a["ab"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(k=P + 8), INVALID),
    (dict(lse=P + 2), INVALID), (dict(B=0), INVALID), (dict(Lq=0), INVALID), (dict(Lk=-1), INVALID),
    (dict(Hq=3, Hkv=2), INVALID), (dict(Hkv=0), INVALID), (dict(d=0), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(causal=2), INVALID), (dict(wl=-2), INVALID), (dict(wr=-5), INVALID),
    (dict(Lq=1 << 20, Hq=64, d=128), INVALID),
    (dict(cap=-1.0), INVALID), (dict(cap=float("nan")), INVALID), (dict(cap=float("inf")), INVALID),
    (dict(al=P + 2), INVALID), (dict(al=P, ab=1), INVALID), (dict(al=P, ab=-2), INVALID),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cq=P, ck=P, B=2, mq=10, mk=10, tq=16, tk=16, Hq=4, Hkv=2,
             d=128, scale=0.1, causal=1, wl=-1, wr=-1, cap=0.0, al=None, ab=0)
    a.update(kw)
    return lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"], a["mq"],
                             a["mk"], a["tq"], a["tk"], a["Hq"], a["Hkv"], a["d"], a["scale"],
                             a["causal"], a["wl"], a["wr"], a["cap"], a["al"], a["ab"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), INVALID), (dict(ck=P + 2), INVALID), (dict(B=0), INVALID),
    (dict(tq=-1), INVALID), (dict(mq=20), INVALID), (dict(mq=0), INVALID), (dict(mk=-1), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(Hq=5), INVALID), (dict(cap=-0.5), INVALID),
    (dict(al=P, ab=3), INVALID),
])
def test_varlen_rejects(lib, kw, code):
    assert varlen(lib, **kw) == code


def varlen_run(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cq=P, ck=P, plan=P, n=2, B=2, mq=10, mk=10, tq=16,
             tk=16, Hq=4, Hkv=2, d=128, scale=0.1, causal=1, wl=-1, wr=-1, cap=0.0, al=None, ab=0)
    a.update(kw)
    return lib.fa_fwd_varlen_run(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                 a["plan"], a["n"], a["B"], a["mq"], a["mk"], a["tq"], a["tk"],
                                 a["Hq"], a["Hkv"], a["d"], a["scale"], a["causal"], a["wl"],
                                 a["wr"], a["cap"], a["al"], a["ab"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(plan=None), INVALID), (dict(plan=P + 4), INVALID), (dict(n=-1), INVALID),
    (dict(n=0), INVALID), (dict(n=0, plan=None), INVALID), (dict(n=3), INVALID),
    (dict(tq=300, mq=300, n=5), INVALID),
    (dict(cq=None), INVALID), (dict(mq=20), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(Hq=5), INVALID), (dict(cap=-0.5), INVALID), (dict(al=P, ab=3), INVALID),
])
def test_varlen_run_rejects(lib, kw, code):
    assert varlen_run(lib, **kw) == code


def test_varlen_run_empty_batch_is_a_noop(lib):
    # total_q = 0: nothing to compute, so no plan item and no launch
    assert varlen_run(lib, tq=0, mq=0, n=0) == OK
    assert varlen_run(lib, tq=0, mq=0, n=0, plan=None) == OK


def test_varlen_empty_batch_is_a_no_op(lib):
    assert varlen(lib, tq=0, mq=0) == OK


def test_workspace_size(lib):
    ws = lib.fa_decode_paged_workspace_size
    # 64 requests, 32 heads, d 128, 512 blocks of 16 tokens, 512-token splits -> 16 splits
    n_o = 64 * 32 * 16 * 128 * 4
    n_l = 64 * 32 * 16 * 4
    n_w = 64 * 16 * 2 * 4      # the device-made work order: one (request, split) pair per slot
    up = lambda x: (x + 255) // 256 * 256
    assert ws(64, 32, 128, 512, 16, 512) == up(n_o) + up(n_l) + up(n_w)
    assert ws(64, 32, 128, 512, 16, 0) == ws(64, 32, 128, 512, 16, 512)
    assert ws(1, 1, 64, 1, 1, 16) == up(64 * 4) + up(4) + up(8)
    for bad in [(0, 32, 128, 512, 16, 0), (1, 32, 96, 4, 16, 0), (1, 32, 128, 4, 16, 24),
                (1, 32, 128, 0, 16, 0), (1, 32, 128, 4, 0, 0), (1, 32, 128, 4, 16, -16)]:
        assert ws(*bad) == 0


def decode(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, sl=P, o=P, lse=P, B=4, Hq=8, Hkv=2, d=128, pages=64, ps=16,
             mb=8, scale=0.1, wl=-1, cap=0.0, al=None, ast=0, split=0, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.fa_decode_paged(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"], a["B"],
                               a["Hq"], a["Hkv"], a["d"], a["pages"], a["ps"], a["mb"], a["scale"],
                               a["wl"], a["cap"], a["al"], a["ast"], a["split"], a["ws"], a["wsb"],
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), INVALID), (dict(sl=P + 1), INVALID), (dict(kc=None), INVALID),
    (dict(pages=0), INVALID), (dict(ps=0), INVALID), (dict(mb=0), INVALID),
    (dict(split=24), INVALID), (dict(split=-16), INVALID), (dict(wl=-2), INVALID),
    (dict(Hkv=3), INVALID), (dict(d=32), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws=P + 16), WORKSPACE), (dict(wsb=1024), WORKSPACE),
    (dict(B=70000), INVALID), (dict(cap=-1.0), INVALID), (dict(cap=math.inf), INVALID),
    (dict(al=P + 2), INVALID), (dict(al=P, ast=3), INVALID),
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


def decode_noalloc(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, sl=P, o=P, lse=P, B=4, Hq=8, Hkv=2, d=128, pages=64, ps=16,
             mb=8, scale=0.1, wl=-1, cap=0.0, al=None, ast=0, split=0)
    a.update(kw)
    return lib.fa_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"],
                                       a["B"], a["Hq"], a["Hkv"], a["d"], a["pages"], a["ps"],
                                       a["mb"], a["scale"], a["wl"], a["cap"], a["al"], a["ast"],
                                       a["split"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), INVALID), (dict(sl=P + 1), INVALID), (dict(kc=None), INVALID),
    (dict(pages=0), INVALID), (dict(split=24), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(Hkv=3), INVALID), (dict(cap=-1.0), INVALID),
    # partials beyond the 32 MiB scratch array: 256 requests x 64 heads x 16 splits x 128 x 4 B
    (dict(B=256, Hq=64, Hkv=8, mb=512), WORKSPACE),
    (dict(B=64, Hq=32, Hkv=8, mb=512, split=16), WORKSPACE),
])
def test_decode_noalloc_rejects_before_any_hip_call(lib, kw, code):
    assert decode_noalloc(lib, **kw) == code


def test_decode_noalloc_limit_matches_workspace_size(lib):
    """The 32 MiB scratch array holds the paged-decode workload's partials (64
    requests, 32 query heads, 8192-token tables, 512-token splits) with room."""
    assert fa.DECODE_NOALLOC_MAX_BYTES == 32 << 20
    need = lib.fa_decode_paged_workspace_size(64, 32, 128, 512, 16, 512)
    assert 0 < need <= fa.DECODE_NOALLOC_MAX_BYTES
    assert lib.fa_decode_paged_workspace_size(256, 64, 128, 512, 16, 512) > fa.DECODE_NOALLOC_MAX_BYTES


def decode_run(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, sl=P, plan=P, n=4, o=P, lse=P, B=4, Hq=8, Hkv=2, d=128,
             pages=64, ps=16, mb=8, scale=0.1, wl=-1, cap=0.0, al=None, ast=0, split=0, ws=P,
             wsb=1 << 30)
    a.update(kw)
    return lib.fa_decode_paged_run(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["plan"], a["n"],
                                   a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                   a["pages"], a["ps"], a["mb"], a["scale"], a["wl"], a["cap"],
                                   a["al"], a["ast"], a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(plan=None), INVALID), (dict(plan=P + 4), INVALID), (dict(n=-1), INVALID),
    # 8 blocks of 16 tokens = 128 keys = one 512-token split per request: at most B items
    (dict(n=5), INVALID), (dict(split=16, n=33), INVALID),
    (dict(bt=None), INVALID), (dict(split=24), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE),
])
def test_decode_run_rejects(lib, kw, code):
    assert decode_run(lib, **kw) == code


def kvcache(lib, **kw):
    a = dict(q=P, kc=P, vc=P, kn=P, vn=P, bt=P, sl=P, o=P, lse=P, B=2, Lq=64, Hq=8, Hkv=2, d=128,
             pages=64, ps=16, mb=8, scale=0.1, causal=1, wl=-1, wr=-1, cap=0.0, al=None, ab=0)
    a.update(kw)
    return lib.fa_fwd_kvcache(a["q"], a["kc"], a["vc"], a["kn"], a["vn"], a["bt"], a["sl"], a["o"],
                              a["lse"], a["B"], a["Lq"], a["Hq"], a["Hkv"], a["d"], a["pages"], a["ps"],
                              a["mb"], a["scale"], a["causal"], a["wl"], a["wr"], a["cap"], a["al"],
                              a["ab"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), INVALID), (dict(vn=None), INVALID), (dict(kn=P + 8), INVALID),
    (dict(bt=None), INVALID), (dict(sl=P + 2), INVALID), (dict(kc=None), INVALID),
    (dict(o=P + 4), INVALID), (dict(B=0), INVALID), (dict(Lq=-1), INVALID),
    (dict(pages=0), INVALID), (dict(mb=0), INVALID), (dict(ps=0), INVALID),
    (dict(ps=8), UNSUPPORTED), (dict(ps=24), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(Hkv=3), INVALID), (dict(scale=float("nan")), INVALID), (dict(causal=5), INVALID),
    (dict(wl=-3), INVALID), (dict(ps=1 << 16, Hkv=64), INVALID), (dict(mb=1 << 26, ps=16), INVALID),
    (dict(cap=-2.0), INVALID), (dict(al=P + 1), INVALID),
    # grid limits, checked before the append is enqueued (no HIP call here)
    (dict(B=70000), INVALID), (dict(B=16384, Lq=(1 << 24) - 64, Hq=1, Hkv=1, d=64), INVALID),
])
def test_kvcache_rejects(lib, kw, code):
    assert kvcache(lib, **kw) == code


def test_kvcache_no_query_rows_is_a_no_op(lib):
    assert kvcache(lib, Lq=0) == OK
    assert kvcache(lib, Lq=0, kn=None, vn=None) == OK


def _golden_cu():
    path = os.path.join(ROOT, "tests", "golden", "cu_seqlens_examples.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lens, cu = line.split("|")
        rows.append(([int(x) for x in lens.split()], [int(x) for x in cu.split()]))
    return rows


@pytest.mark.parametrize("lens,cu", _golden_cu())
def test_cu_seqlens_worked_examples(lens, cu):
    if lens:
        assert fa.cu_seqlens_from_lengths(lens).tolist() == cu
    assert fa.cu_seqlens_from_lengths(fa.lengths_from_cu_seqlens(cu)).tolist() == cu
    assert fa.lengths_from_cu_seqlens(cu).sum() == cu[-1]


def test_cu_seqlens_rejects_bad_input():
    with pytest.raises(ValueError):
        fa.cu_seqlens_from_lengths([3, -1])
    with pytest.raises(ValueError):
        fa.lengths_from_cu_seqlens([1, 4])
    with pytest.raises(ValueError):
        fa.lengths_from_cu_seqlens([0, 5, 3])


def test_binding_requires_device_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


def test_no_oracle_import_in_product():
    """The product package never imports or references the oracle."""
    pkg = os.path.join(ROOT, "exact_attention_17_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt, f


def bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=2, Lq=100, Lk=130, Hq=4, Hkv=2,
             d=128, scale=0.1, causal=1, wl=-1, wr=-1, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                      a["B"], a["Lq"], a["Lk"], a["Hq"], a["Hkv"], a["d"], a["scale"], a["causal"],
                      a["wl"], a["wr"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(do=None), INVALID),
    (dict(dq=None), INVALID), (dict(dk=P + 8), INVALID), (dict(dv=P + 2), INVALID),
    (dict(lse=P + 2), INVALID), (dict(B=0), INVALID), (dict(Lq=0), INVALID), (dict(Lk=0), INVALID),
    (dict(Hq=5), INVALID), (dict(d=96), UNSUPPORTED), (dict(scale=float("nan")), INVALID),
    (dict(causal=3), INVALID), (dict(wl=-2), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws=P + 64), WORKSPACE), (dict(wsb=1000), WORKSPACE),
    (dict(B=1 << 14, Lq=1 << 15, Hq=4), INVALID),        # statistics beyond 2^31 bytes
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_bwd_workspace_size(lib):
    # per (batch, head): rows padded to 128, two floats each
    assert lib.fa_bwd_workspace_size(2, 4, 100) == 2 * 4 * 128 * 2 * 4
    assert lib.fa_bwd_workspace_size(1, 1, 129) == 256 * 2 * 4
    assert lib.fa_bwd_workspace_size(0, 4, 100) == 0
    assert lib.fa_bwd_workspace_size(1 << 14, 4, 1 << 15) == 0


def bwd_varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, cq=P, ck=P, B=2, mq=10, mk=10,
             tq=16, tk=16, Hq=4, Hkv=2, d=128, scale=0.1, causal=1, wl=-1, wr=-1, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                             a["dv"], a["cq"], a["ck"], a["B"], a["mq"], a["mk"], a["tq"], a["tk"],
                             a["Hq"], a["Hkv"], a["d"], a["scale"], a["causal"], a["wl"], a["wr"],
                             a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(do=None), INVALID),
    (dict(dq=P + 8), INVALID), (dict(cq=None), INVALID), (dict(ck=P + 2), INVALID),
    (dict(B=0), INVALID), (dict(tq=-1), INVALID), (dict(mq=20), INVALID), (dict(mk=-1), INVALID),
    (dict(Hq=5), INVALID), (dict(d=96), UNSUPPORTED), (dict(wr=-3), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws=P + 32), WORKSPACE), (dict(wsb=100), WORKSPACE),
])
def test_bwd_varlen_rejects(lib, kw, code):
    assert bwd_varlen(lib, **kw) == code


def test_bwd_varlen_workspace_size(lib):
    # rows: (total_q / 128 + B) tile slots of 128 per head, two floats each
    assert lib.fa_bwd_varlen_workspace_size(2, 4, 16) == 4 * (0 + 2) * 128 * 2 * 4
    assert lib.fa_bwd_varlen_workspace_size(3, 2, 300) == 2 * (2 + 3) * 128 * 2 * 4
    assert lib.fa_bwd_varlen_workspace_size(0, 4, 16) == 0
    # nothing to do: both totals 0 is accepted without a launch
    assert bwd_varlen(lib, tq=0, tk=0, mq=0, mk=0) == OK


def test_membw_probe_rejects_bad_arguments():
    """The benchmark's read-bandwidth probe (its own library) validates its
    arguments on the host and enqueues nothing when they are bad."""
    from exact_attention_17_amd import build
    if not os.path.exists(build.MEMBW_LIB_PATH):
        build.build_library(membw=True)
    lib = ctypes.CDLL(build.MEMBW_LIB_PATH)
    fn = lib.fa_membw_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    for src, nbytes, sink, blocks in [(None, 16, P, 1), (P, 0, P, 1), (P, 24, P, 1), (P + 8, 16, P, 1),
                                      (P, 16, None, 1), (P, 16, P + 2, 1), (P, 16, P, 0)]:
        assert fn(src, nbytes, sink, blocks, None) == 1
