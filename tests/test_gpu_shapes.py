"""GPU parity on the less common shapes the kernels have separate arithmetic for:
page sizes that are not a power of two (the page-table lookup then takes the
multiply-high division instead of a shift and mask), block sizes that are not a power of
two (the block index of a list slot then takes a 32-bit division), padded pages on
several layers, and key lists long enough for the largest split counts
("QSASparseAttentionRaggedPaged", Tensor shapes; "Struct_msa_attention_ragged_paged",
Args; "latent_sparse_attention_ragged_paged", Args)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(case, options=None):
    dc = D.to_device(case, DEV)
    out = D.run(dc, options=options)
    torch.cuda.synchronize()
    return out, oracle.run_case(case)


@pytest.mark.parametrize("ps", [48, 96])
@pytest.mark.parametrize("g,d", [(4, 128), (16, 128), (2, 64)])
def test_index_selected_page_size_not_power_of_two(ps, g, d):
    case = W.make_qsa(name="ps_npow2", seed=100 + ps + g, rows=[1, 3, 1, 2], cache_lengths=[700, 130, 47, 1000],
                      page_size=ps, num_layers=2, layer_idx=1, num_kv_heads=2, group=g, head_dim=d, dtype="bf16",
                      out_dtype="f32", selection_width=300, selection="uniform_counts", scale=1 / np.sqrt(d),
                      page_pad=64)
    announce("index-selected page %d group %d d %d" % (ps, g, d))
    got, ref = run(case)
    compare(got, ref, "bf16", "page %d g=%d d=%d" % (ps, g, d))


@pytest.mark.parametrize("dtype,g", [("e4m3", 8), ("bf16", 4), ("bf16", 16)])
def test_block_sparse_block_size_not_power_of_two(dtype, g):
    """Blocks of 24 keys in pages of 96 (a block never straddles a page): the block
    index of a list slot is a division, and the page lookup a multiply-high."""
    case = W.make_block_sparse(name="bs_npow2", seed=110 + g, cache_lengths=[900, 2000, 300, 140], rows=[1, 2, 1, 1],
                               page_size=96, num_kv_heads=2, group=g, head_dim=128, dtype=dtype, topk=6, block_size=24,
                               scale=1 / np.sqrt(128), std=0.5)
    announce("block-sparse block 24 page 96 %s g=%d" % (dtype, g))
    got, ref = run(case)
    compare(got, ref, dtype, "block 24 %s g=%d" % (dtype, g))


def test_latent_page_sizes_not_power_of_two():
    case = W.make_latent(name="latent_npow2", seed=120, decode_positions=[700, 2100, 333], prefill_positions=[900],
                         prefill_rows=5, num_heads=32, head_dim=128, dtype="bf16", out_dtype="f32", window=40,
                         swa_page_size=48, comp_page_size=24, num_comp=60, comp_ratio=4, unused_frac=0.1,
                         scale=1 / np.sqrt(128))
    announce("latent window page 48, compressed page 24")
    got, ref = run(case)
    compare(got, ref, "bf16", "latent pages 48/24")


@pytest.mark.parametrize("g", [4, 16])
def test_index_selected_long_lists(g):
    """Two decode rows selecting 40001 and 65536 keys (width 65536): each list is split
    the planner's way and 64 ways, the largest split count."""
    case = W.make_qsa(name="long", seed=130 + g, rows=[1, 1], cache_lengths=[40000, 70000], page_size=128,
                      num_layers=1, layer_idx=0, num_kv_heads=2, group=g, head_dim=128, dtype="bf16", out_dtype="f32",
                      selection_width=65536, selection="min", scale=1 / np.sqrt(128))
    announce("index-selected lists of up to 65536 keys, group %d" % g)
    got, ref = run(case)
    compare(got, ref, "bf16", "long lists g=%d" % g)
    got64, _ = run(case, options={"num_splits": 64})
    compare(got64, ref, "bf16", "long lists g=%d, 64 splits" % g)


def test_block_sparse_long_lists():
    """512 blocks of 64 keys per (kv head, row): 32768 keys each."""
    case = W.make_block_sparse(name="bs_long", seed=140, cache_lengths=[40000, 33000], rows=[1, 1], page_size=128,
                               num_kv_heads=2, group=8, head_dim=128, dtype="e4m3", topk=512, block_size=64,
                               scale=1 / np.sqrt(128), std=0.5)
    announce("block-sparse 512 blocks of 64")
    got, ref = run(case)
    compare(got, ref, "e4m3", "block-sparse 512 blocks")
