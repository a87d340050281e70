"""HIP graph capture of the entry points.

Every call launches on the caller's stream and allocates, frees or
synchronises nothing, so a sequence of calls on preallocated buffers can be
captured into a HIP graph and replayed.  Each test captures such a sequence,
then replays it several times with unrelated eager work, a clobber of the
outputs and a synchronisation between replays, and checks every replay
bitwise against the eager result."""

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_compare(g, outs, refs, replays=3):
    scratch = torch.randn(1 << 20, device="cuda")
    for _ in range(replays):
        for o in outs:
            o.fill_(7)                                  # results must come from the replay
        scratch.mul_(1.0001).add_(0.5)                  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r)


def test_graph_dense_and_varlen_forward(fa):
    w = workloads.random_dense(61, 2, 700, 700, 8, 2, 128, True, (300, 0))
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o, lse = torch.empty_like(q), torch.empty((2, 8, 700), dtype=torch.float32, device="cuda")
    ref = [t.clone() for t in fa.fa_fwd(q, k, v, w.scale, True, (300, 0))]
    g = capture(lambda: fa.fa_fwd(q, k, v, w.scale, True, (300, 0), out=o, lse=lse))
    replay_and_compare(g, [o, lse], ref)

    vw = workloads.random_varlen(62, [300, 1, 1000, 129], 4, 2, 64, True, (200, 0))
    qv, kv, vv = dev(vw.q), dev(vw.k), dev(vw.v)
    cu = dev(torch.from_numpy(vw.cu_seqlens))
    plan = dev(torch.from_numpy(np.ascontiguousarray(
        fa.fa_varlen_plan(vw.cu_seqlens, vw.cu_seqlens, True, (200, 0)))))
    ov, lv = torch.empty_like(qv), torch.empty((4, qv.shape[0]), dtype=torch.float32, device="cuda")
    ov2, lv2 = torch.empty_like(qv), torch.empty_like(lv)
    r1 = [t.clone() for t in fa.fa_fwd_varlen(qv, kv, vv, cu, cu, vw.max_seqlen, vw.max_seqlen,
                                              vw.scale, True, (200, 0))]

    def both():
        fa.fa_fwd_varlen(qv, kv, vv, cu, cu, vw.max_seqlen, vw.max_seqlen, vw.scale, True, (200, 0),
                         out=ov, lse=lv)
        fa.fa_fwd_varlen_run(qv, kv, vv, cu, cu, plan, vw.max_seqlen, vw.max_seqlen, vw.scale, True,
                             (200, 0), out=ov2, lse=lv2)
    g = capture(both)
    replay_and_compare(g, [ov, lv, ov2, lv2], r1 + r1)


def test_graph_paged_decode_and_chunked_prefill(fa):
    p = workloads.random_paged(63, [900, 17, 1500, 0], 32, 8, 128, 16, 200, 512, max_blocks=100)
    q, kc, vc = dev(p.q), dev(p.k_cache), dev(p.v_cache)
    bt, sl = dev(torch.from_numpy(p.block_table)), dev(torch.from_numpy(p.seqlens))
    ws = torch.empty(fa.fa_decode_paged_workspace_size(4, 32, 128, 100, 16, 512), dtype=torch.uint8,
                     device="cuda")
    plan = dev(torch.from_numpy(np.ascontiguousarray(fa.fa_decode_plan(p.seqlens, 16, 100, -1, 512))))
    o1, l1 = torch.empty_like(q), torch.empty((4, 32), dtype=torch.float32, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    ref = [t.clone() for t in fa.fa_decode_paged(q, kc, vc, bt, sl, p.scale, -1, 512, workspace=ws)]

    def both():
        fa.fa_decode_paged(q, kc, vc, bt, sl, p.scale, -1, 512, out=o1, lse=l1, workspace=ws)
        fa.fa_decode_paged_run(q, kc, vc, bt, sl, plan, p.scale, -1, 512, out=o2, lse=l2, workspace=ws)
    g = capture(both)
    replay_and_compare(g, [o1, l1, o2, l2], ref + ref)

    c = workloads.random_kvcache(64, [300, 0, 777], 100, 8, 2, 128, 16)
    qc, kcc, vcc = dev(c.q), dev(c.k_cache), dev(c.v_cache)
    btc, slc = dev(torch.from_numpy(c.block_table)), dev(torch.from_numpy(c.cache_seqlens))
    kn, vn = dev(c.k_new), dev(c.v_new)
    oc, lc = torch.empty_like(qc), torch.empty((3, 8, 100), dtype=torch.float32, device="cuda")
    refc = [t.clone() for t in fa.fa_fwd_kvcache(qc, kcc, vcc, btc, slc, kn, vn, c.scale, True)]
    # the append writes the same rows on every call, so replays see the same cache
    g = capture(lambda: fa.fa_fwd_kvcache(qc, kcc, vcc, btc, slc, kn, vn, c.scale, True, out=oc, lse=lc))
    replay_and_compare(g, [oc, lc], refc)


def test_graph_backward(fa):
    w = workloads.random_dense(65, 1, 600, 600, 8, 2, 128, True, (-1, -1))
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o, lse = fa.fa_fwd(q, k, v, w.scale, True)
    do = workloads.device_normal(66, tuple(q.shape), "cuda")
    ws = torch.empty(fa.fa_bwd_workspace_size(1, 8, 600), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ref = [t.clone() for t in fa.fa_bwd(q, k, v, o, lse, do, w.scale, True, workspace=ws)]
    g = capture(lambda: fa.fa_bwd(q, k, v, o, lse, do, w.scale, True, dq=dq, dk=dk, dv=dv, workspace=ws))
    replay_and_compare(g, [dq, dk, dv], ref)

