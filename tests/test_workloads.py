"""Input generators: determinism and the structure the workload recipes promise."""
import numpy as np
import torch

import workloads as W


def test_deterministic():
    a, b = W.c1_tiny_fp32(), W.c1_tiny_fp32()
    assert torch.equal(a.q.view(torch.uint8), b.q.view(torch.uint8)) if a.q.dtype != torch.float32 \
        else torch.equal(a.q, b.q)
    assert np.array_equal(a.token_indices, b.token_indices)
    assert np.array_equal(a.kv.lookup_table, b.kv.lookup_table)
    assert torch.equal(a.kv.storage.isnan(), b.kv.storage.isnan())


def test_c1_recipe():
    c = W.c1_tiny_fp32()
    assert list(np.diff(c.input_row_offsets)) == [3, 5]
    assert list(c.kv.cache_lengths) == [29, 59]
    assert c.kv.num_pages == 6 + 4 and c.kv.page_size == 16
    pos = c.positions()
    for r in range(c.total_q):
        n = c.counts[r]
        assert 1 <= n <= min(16, pos[r] + 1)
        sel = c.token_indices[r, :n]
        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] <= pos[r]
        assert (c.token_indices[r, n:] == -7).all()


def test_unreadable_slots_are_nan():
    c = W.make_qsa(seed=3, rows=[2], cache_lengths=[5], page_size=4, num_layers=2, layer_idx=1,
                   num_kv_heads=1, group=1, head_dim=4, dtype="bf16", out_dtype="bf16",
                   selection_width=4, selection="min", scale=1.0, spare_pages=1)
    pv = c.kv.pages_view()
    assert pv[:, :, 0].isnan().all()                       # other layer
    lut = c.kv.lookup_table[0]
    assert not pv[int(lut[0]), :, 1].isnan().any()          # positions 0..3
    assert not pv[int(lut[1]), :, 1, :3].isnan().any()      # positions 4..6
    assert pv[int(lut[1]), :, 1, 3].isnan().all()           # position 7 > last position 6


def test_block_sparse_recipe():
    c = W.make_block_sparse(seed=4, cache_lengths=[300, 129], page_size=128, num_kv_heads=2, group=4,
                            head_dim=8, dtype="e4m3", topk=3, block_size=64, scale=0.1)
    pos = c.positions()
    for g in range(2):
        for r in range(2):
            ids = c.d_indices[g, r]
            assert len(set(ids.tolist())) == 3 and pos[r] // 64 in ids and ids.max() == pos[r] // 64


def test_gathered_bytes():
    c = W.c1_tiny_fp32()
    assert W.gathered_kv_bytes(c) == int(c.counts.sum()) * 1 * 2 * 64 * 4


def test_compress_recipe():
    c = W.make_compress(seed=5, cache_lengths=[9, 0], rows=[1, 3], page_size=4, num_layers=2, layer_idx=0,
                        head_dim=8, dtype="bf16", ratio=4, rotary_dim=4)
    assert c.key_counts.tolist() == [10, 3] and c.max_blocks == 3
    assert c.blocks_per_sequence().tolist() == [2, 0]
    pv = c.kv.pages_view()
    assert pv[:, 1].isnan().all() and pv[:, :, 1].isnan().all()      # V plane, other layer
    lut = c.kv.lookup_table[0]
    assert not pv[int(lut[2]), 0, 0, :2].isnan().any() and pv[int(lut[2]), 0, 0, 2:].isnan().all()
    f = c.freqs.double()
    assert c.freqs.shape == (12, 4) and torch.allclose(f[:, 0::2] ** 2 + f[:, 1::2] ** 2,
                                                       torch.ones(12, 2, dtype=torch.float64), atol=1e-6)
    # 2 blocks x 4 keys x 16 B + 2 written x 16 B + 2 table rows x 16 B + gamma 16 B + 2 counts + 2 lut entries
    assert W.compress_bytes(c) == 128 + 32 + 32 + 16 + 8 + 8


def test_select_recipe():
    c = W.make_select(seed=6, rows=[2, 1], cache_lengths=[9, 0], head_dim=8, dtype="bf16", ratio=4, topk=2,
                      integer=True)
    assert c.max_blocks == 2 and c.W == 11
    assert c.positions().tolist() == [9, 10, 0] and c.candidates().tolist() == [2, 2, 0]
    bk = c.block_keys.view(2, 2, 8)
    assert not bk[0].isnan().any() and bk[1].isnan().all()          # sequence 1 has no complete block
    v = c.q_index.float()
    assert (v == v.round()).all() and v.abs().max() <= 2
