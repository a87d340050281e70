"""GPU parity at the size limits of the boundary (sampled outputs).

* Dense prefill with Lq * Hq * d = 2^30 - 2048 elements per batch, the
  largest the library accepts (it addresses a batch with 32-bit byte
  offsets): rows at the start, in the middle and at the very end, and the
  backward on sampled rows and keys.
* Paged decode over a page pool of more than 2^32 bytes per cache, with the
  requests' pages at the top of the pool (64-bit page offsets).

Inputs are drawn on the device by a seeded generator (workloads.device_normal)
and copied to the host for the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from bwd_tolerance import key_rows_tolerance, query_rows_tolerance, ratio
from gpu_helpers import bits, check, f64

pytestmark = pytest.mark.gpu


def test_dense_at_the_per_batch_limit(fa):
    Hq, Hkv, d = 16, 4, 128
    L = (1 << 30) // (Hq * d) - 1                  # 524287 rows: Lq * Hq * d = 2^30 - 2048
    assert L * Hq * d < (1 << 30)
    scale = 1.0 / math.sqrt(d)
    q = workloads.device_normal(71, (1, L, Hq, d))
    k = workloads.device_normal(72, (1, L, Hkv, d))
    v = workloads.device_normal(73, (1, L, Hkv, d))
    o, lse = fa.fa_fwd(q, k, v, scale, True)
    dout = workloads.device_normal(74, (1, L, Hq, d))
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, dout, scale, True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 262143, 262144, L - 129, L - 128, L - 2, L - 1])
    keys = np.array([L - 300, L - 129, L - 64, L - 2, L - 1])
    # host copies of what the oracle reads (heads 0 and 13, KV heads 0 and 3)
    qb, kb, vb, db = (bits(t.cpu()) for t in (q, k, v, dout))
    o_rows = f64(o[0, rows].cpu())
    lse_rows = f64(lse[0, :, rows].cpu())
    for h in (0, 13):
        O, LSE = oracle.attention_rows_ref(qb, kb, vb, 0, h, rows, scale, True)
        check(f"limit fwd h{h}", o_rows[:, h], lse_rows[h], O, LSE)
        ref = oracle.attention_bwd_query_rows_ref(qb, kb, vb, db, 0, h, rows, scale, True)
        tol = query_rows_tolerance(qb, kb, vb, db, 0, h, rows, scale, True, (-1, -1), ref)
        x = ratio(f64(dq[0, rows, h].cpu()), ref, tol)
        print(f"[parity] limit bwd dq h{h}: max err/tol {x:.3f}", flush=True)
        assert x <= 1.0
    for g in (0, 3):
        rk, rv = oracle.attention_bwd_key_rows_ref(qb, kb, vb, db, 0, g, keys, scale, True,
                                                   row_start=int(keys.min()))
        tk, tv = key_rows_tolerance(qb, kb, vb, db, 0, g, keys, scale, True, (-1, -1), rk, rv,
                                    row_start=int(keys.min()))
        xk, xv = ratio(f64(dk[0, keys, g].cpu()), rk, tk), ratio(f64(dv[0, keys, g].cpu()), rv, tv)
        print(f"[parity] limit bwd dk/dv g{g}: max err/tol {xk:.3f} / {xv:.3f}", flush=True)
        assert xk <= 1.0 and xv <= 1.0


def test_decode_with_a_pool_beyond_4_gib(fa):
    Hq, Hkv, d, ps = 16, 8, 128, 16
    pages = 280000                                 # 280000 * 16 * 8 * 128 * 2 B = 9.2 GB per cache
    assert pages * ps * Hkv * d * 2 > (1 << 32)
    lens = np.array([1000, 1, 4097, 300], dtype=np.int32)
    need = -(-lens // ps)
    max_blocks = int(need.max())
    # the requests' pages are the last ids of the pool, in reverse order
    table = np.zeros((len(lens), max_blocks), dtype=np.int32)
    nxt = pages - 1
    for b, n in enumerate(need):
        table[b, :n] = np.arange(nxt, nxt - n, -1)
        nxt -= n
    kc = workloads.device_normal(81, (pages, ps, Hkv, d))
    vc = workloads.device_normal(82, (pages, ps, Hkv, d))
    q = workloads.device_normal(83, (len(lens), 1, Hq, d))
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(lens).cuda()
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fa_decode_paged(q, kc, vc, bt, sl, scale, -1, 512)
    torch.cuda.synchronize()
    used = np.unique(table[table > 0])
    # the oracle reads the used pages only: copy them into a small pool and remap the table
    small_k = bits(kc[torch.from_numpy(used).cuda()].cpu())
    small_v = bits(vc[torch.from_numpy(used).cuda()].cpu())
    remap = {int(p): i for i, p in enumerate(used)}
    small_table = np.vectorize(lambda x: remap.get(int(x), 0))(table).astype(np.int32)
    O, LSE = oracle.decode_paged_ref(bits(q.cpu()), small_k, small_v, small_table, lens, ps, scale)
    check("decode pool > 4 GiB", o.cpu(), lse.cpu(), O, LSE)
