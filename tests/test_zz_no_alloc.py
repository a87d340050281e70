"""fa_decode_paged_noalloc (the allocation-free paged decode: split partials in
the library's per-GPU scratch array) against fa_decode_paged with a caller
workspace: two calls in a row, the second with a smaller batch, each bitwise
equal to the workspace call and within the oracle tolerance."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bits, check, dev

pytestmark = pytest.mark.gpu


def test_noalloc_decode_matches_workspace_call(fa):
    cases = [
        # lengths, Hq, Hkv, d, page_size, pool pages, split
        ([3000, 17, 900, 4096, 1, 2500], 32, 8, 128, 16, 1200, 512),   # head-set kernel
        ([700, 33], 8, 1, 64, 24, 80, 256),                            # general kernel, odd page size
    ]
    for i, (lens, Hq, Hkv, d, ps, pool, split) in enumerate(cases):
        p = workloads.random_paged(600 + i, lens, Hq, Hkv, d, ps, pool, split)
        q, kc, vc = dev(p.q), dev(p.k_cache), dev(p.v_cache)
        bt, sl = dev(torch.from_numpy(p.block_table)), dev(torch.from_numpy(p.seqlens))
        ref_o, ref_l = fa.fa_decode_paged(q, kc, vc, bt, sl, p.scale, -1, split)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], Hq), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        o, l = fa.fa_decode_paged_noalloc(q, kc, vc, bt, sl, p.scale, -1, split, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() <= before      # nothing allocated through torch
        assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
        print(f"[noalloc] call {i}: batch {len(lens)}, Hq {Hq}, d {d}", flush=True)
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(l, ref_l)
        O, LSE = oracle.decode_paged_ref(bits(p.q), bits(p.k_cache), bits(p.v_cache), p.block_table,
                                         p.seqlens, p.page_size, p.scale)
        check(f"noalloc{i}", o, l, O, LSE)


def test_noalloc_decode_rejects_oversized_call(fa):
    p = workloads.random_paged(610, [100], 64, 8, 128, 16, 600, 16, max_blocks=600)
    q, kc, vc = dev(p.q), dev(p.k_cache), dev(p.v_cache)
    q = q.repeat(300, 1, 1, 1).contiguous()
    bt = dev(torch.from_numpy(np.repeat(p.block_table, 300, axis=0)))
    sl = dev(torch.from_numpy(np.repeat(p.seqlens, 300)))
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_paged_noalloc(q, kc, vc, bt, sl, p.scale, -1, 16)
    assert e.value.status == 3
