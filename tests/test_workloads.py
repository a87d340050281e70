"""The seeded generators reproduce the workload statistics derived for them
(sum of decode context lengths, page counts, varlen lengths), so a change in
draw order or recipe is caught on the CPU."""

import numpy as np
import torch

import workloads


def test_paged_decode_layout_statistics():
    lens, table, used, spare = workloads.paged_decode_layout()
    assert lens.shape == (64,) and lens.min() >= 512 and lens.max() <= 8192
    assert int(lens.sum()) == 311415
    assert int(lens.min()) == 977 and int(lens.max()) == 8071
    assert used == 19492
    npages = -(-lens.astype(np.int64) // 16)
    # 512-token splits: 641 of them are non-empty
    assert int((-(-lens.astype(np.int64) // 512)).sum()) == 641
    ids = np.concatenate([table[b, :npages[b]] for b in range(64)])
    assert len(np.unique(ids)) == used and spare not in ids
    assert (table[0, npages[0]:] == spare).all()
    assert table.shape == (64, 512)


def test_varlen_lengths_and_total():
    lens = np.rint(np.exp(np.random.default_rng(5).uniform(np.log(64), np.log(8192), 16))).astype(int)
    assert lens.tolist() == [3180, 3226, 780, 256, 83, 411, 464, 80, 81, 8159, 1517, 200, 528,
                             7228, 4986, 3847]
    assert lens.sum() == 35026


def test_small_paged_nan_rules():
    w = workloads.random_paged(9, [5, 16, 17], Hq=4, Hkv=2, d=64, page_size=16, pool_pages=8)
    assert torch.isnan(w.k_cache[w.extra["spare_page"]].float()).all()
    last = int(w.block_table[0, 0])
    assert torch.isnan(w.k_cache[last, 5:].float()).all()
    assert not torch.isnan(w.k_cache[last, :5].float()).any()
    full = int(w.block_table[1, 0])
    assert not torch.isnan(w.v_cache[full].float()).any()


def test_bf16_rounding_is_rne():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32)   # exact ties
    y = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert y[0] == 1.0 and y[1] == 1.0 + 2 ** -6
