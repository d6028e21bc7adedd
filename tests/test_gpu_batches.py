"""GPU parity at batch sizes that take each path of the in-kernel row -> sequence
lookup ("QSASparseAttentionRaggedPaged", Tensor shapes: input_row_offsets [batch + 1]):
up to 64 sequences one round of 64 lanes covers, 65 to 1024 several rounds, more than
1024 a binary search over the offsets. Empty sequences (no rows this step) are mixed in,
so rows sit at sequence boundaries of every kind. Each kernel family that looks a row's
sequence up is covered: the wavefront and matrix-core gathers over index lists, the
block-sparse gather (which also needs the row's position), the dense shared-tile kernel,
the latent kernel and the block selection."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
BATCHES = [150, 1500]


def rows_and_cache(batch, seed, max_rows=2, lo=1, hi=120):
    """0..max_rows rows per sequence (some empty, at least one row in all) and cache lengths."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, max_rows + 1, size=batch)
    rows[batch // 2] = max(int(rows[batch // 2]), 1)
    rows[-1] = 0                                  # an empty last sequence
    cache = rng.integers(lo, hi, size=batch, endpoint=True)
    return [int(x) for x in rows], [int(x) for x in cache]


def run(case, options=None):
    dc = D.to_device(case, DEV)
    out = D.run(dc, options=options)
    torch.cuda.synchronize()
    return out, oracle.run_case(case)


@pytest.mark.parametrize("batch", BATCHES)
@pytest.mark.parametrize("g,d", [(4, 128), (16, 64)])
def test_index_selected_many_sequences(batch, g, d):
    rows, cache = rows_and_cache(batch, seed=batch + g)
    case = W.make_qsa(name="many_qsa", seed=batch + g, rows=rows, cache_lengths=cache, page_size=16,
                      num_layers=1, layer_idx=0, num_kv_heads=2, group=g, head_dim=d, dtype="bf16",
                      out_dtype="f32", selection_width=48, selection="uniform_counts", scale=1 / np.sqrt(d))
    announce("index-selected, %d sequences (%d rows), group %d" % (batch, case.total_q, g))
    got, ref = run(case)
    compare(got, ref, "bf16", "index-selected batch=%d g=%d" % (batch, g))


@pytest.mark.parametrize("batch", BATCHES)
def test_block_sparse_many_sequences(batch):
    rows, cache = rows_and_cache(batch, seed=batch + 7, lo=48, hi=200)
    case = W.make_block_sparse(name="many_bs", seed=batch + 7, cache_lengths=cache, rows=rows, page_size=16,
                               num_kv_heads=2, group=8, head_dim=128, dtype="e4m3", topk=3, block_size=16,
                               scale=1 / np.sqrt(128), std=0.5)
    announce("block-sparse, %d sequences (%d rows)" % (batch, case.total_q))
    got, ref = run(case)
    compare(got, ref, "e4m3", "block-sparse batch=%d" % batch)


@pytest.mark.parametrize("batch", BATCHES)
def test_dense_many_sequences(batch):
    rows, _ = rows_and_cache(batch, seed=batch + 11, max_rows=5)
    case = W.make_dense(name="many_dense", seed=batch + 11, rows=rows, num_kv_heads=2, group=8, head_dim=128,
                        dtype="bf16", out_dtype="f32", causal=True, window=-1, scale=1 / np.sqrt(128))
    announce("dense, %d sequences (%d rows)" % (batch, case.total_q))
    got, ref = run(case)
    compare(got, ref, "bf16", "dense batch=%d" % batch)


@pytest.mark.parametrize("batch", BATCHES)
def test_latent_many_sequences(batch):
    rng = np.random.default_rng(batch + 13)
    pos = rng.integers(300, 900, size=batch, endpoint=True)
    case = W.make_latent(name="many_latent", seed=batch + 13, decode_positions=pos[:-2], prefill_positions=pos[-2:],
                         prefill_rows=3, num_heads=32, head_dim=128, dtype="bf16", out_dtype="f32", window=16,
                         swa_page_size=16, comp_page_size=16, num_comp=40, comp_ratio=4, unused_frac=0.1,
                         scale=1 / np.sqrt(128))
    announce("latent, %d sequences (%d rows)" % (batch, case.total_q))
    got, ref = run(case)
    compare(got, ref, "bf16", "latent batch=%d" % batch)


@pytest.mark.parametrize("batch", BATCHES)
def test_selection_many_sequences(batch):
    rows, cache = rows_and_cache(batch, seed=batch + 17, lo=64, hi=400)
    case = W.make_select(name="many_select", seed=batch + 17, rows=rows, cache_lengths=cache, head_dim=64,
                         dtype="bf16", ratio=4, topk=8, integer=True)
    announce("selection, %d sequences (%d rows)" % (batch, case.total_q))
    dc = D.select_to_device(case, DEV)
    idx = torch.full((case.total_q, case.W), -7, dtype=torch.int32, device=DEV)
    counts = torch.full((case.total_q,), -7, dtype=torch.int32, device=DEV)
    blocks = torch.full((case.total_q, case.topk), -7, dtype=torch.int32, device=DEV)
    D.run_select(dc, token_indices=idx, counts=counts, blocks=blocks)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    got_idx, got_counts, got_blocks = idx.cpu().numpy(), counts.cpu().numpy(), blocks.cpu().numpy()
    assert np.array_equal(got_counts, ref[1]), "counts differ"
    for r in range(case.total_q):
        n = ref[1][r]
        assert np.array_equal(got_idx[r, :n], ref[0][r, :n]), "row %d: token indices differ" % r
        assert (got_idx[r, n:] == -7).all(), "row %d: wrote past the count" % r
    assert np.array_equal(got_blocks, ref[2]), "block ids differ"
