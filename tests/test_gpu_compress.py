"""GPU parity of key compression (block keys pooled from the raw index keys of a paged
indexer cache) against the fp64 oracle: both key types, both rotary-table types, every
team width (16- to 1024-byte rows), ratios with a compile-time row count (1, 2, 4, 8,
16) and others, ratios that do and do not divide the page size, blocks that span
pages (also ratios above the page size), padded pages, no rotation and full-width rotation, sequences
with fewer keys than one group, the max_blocks cap, the launch bound from the maximum
cache and prompt lengths, raw keys past the complete groups set to NaN, page-table
entries outside the pool, and the full-size indexer workload.

Tolerance: fp32 block keys within 1e-4; bf16 block keys within max(2e-2, |ref| / 256),
one bf16 rounding (at most |ref| / 512) plus fp32 arithmetic, since RMS-normalised
keys times gamma reach magnitudes of 8 and more where a bf16 step exceeds 2e-2. Rows
that a call does not produce must keep the values the caller left in them."""
import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
CANARY = 1024.0            # exact in bf16 and fp32, far above any block key


def check(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str, canary=CANARY):
    g = to64(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    dead = np.isnan(ref).all(axis=1)
    assert (g[dead] == canary).all(), "%s: %d rows that must stay untouched were written" % (
        what, int((g[dead] != canary).any(axis=1).sum()))
    live = ~dead
    err = np.abs(g[live] - ref[live])
    tol = 1e-4 if dtype == "f32" else np.maximum(2e-2, np.abs(ref[live]) / 256)
    assert np.isfinite(g[live]).all(), what + ": non-finite block keys"
    bad = err > tol
    assert not bad.any(), "%s: %d of %d values off (max abs err %.3e)" % (what, int(bad.sum()), bad.size,
                                                                         float(err.max()))
    return float(err.max()) if err.size else 0.0


def run(case, kv_override=None, mpl=None):
    dc = D.compress_to_device(case, DEV)
    if kv_override:
        for k, v in kv_override.items():
            setattr(dc.kv, k, v)
    out = torch.full((case.batch * case.max_blocks, case.head_dim), CANARY, dtype=W.TORCH_DTYPE[case.dtype],
                     device=DEV)
    import sparse_attention_ragged_amd as qsa
    qsa.compress_keys(dc.kv, dc.key_counts, dc.gamma, dc.freqs, case.layer_idx, case.ratio, case.rotary_dim,
                      case.eps, max_blocks=case.max_blocks,
                      max_prompt_length=case.max_prompt_length if mpl is None else mpl, out=out)
    torch.cuda.synchronize()
    return out


SHAPES = [
    # dtype, freq dtype, head_dim, ratio, rotary_dim, page_size, page_pad
    ("bf16", "f32", 128, 4, 64, 128, 0),
    ("bf16", "bf16", 128, 4, 128, 16, 0),
    ("f32", "f32", 64, 3, 32, 8, 4),
    ("bf16", "f32", 256, 1, 0, 32, 0),
    ("f32", "bf16", 256, 8, 256, 64, 0),
    ("bf16", "f32", 512, 2, 64, 16, 0),
    ("bf16", "f32", 32, 4, 16, 8, 8),
    ("f32", "f32", 16, 5, 16, 4, 0),
    ("bf16", "f32", 8, 2, 8, 4, 0),
    ("f32", "f32", 128, 6, 100, 32, 0),
    ("bf16", "f32", 128, 8, 64, 4, 0),            # ratio above the page size: blocks span 2 pages
]


@pytest.mark.parametrize("dtype,fdt,d,ratio,rd,ps,pad", SHAPES)
def test_compress_matches_oracle(dtype, fdt, d, ratio, rd, ps, pad):
    case = W.make_compress(name="compress_t", seed=61, cache_lengths=[0, 37, 200, 3, 1000, 511],
                           rows=[2, 1, 5, 0, 1, 1], page_size=ps, num_layers=3, layer_idx=2, head_dim=d,
                           dtype=dtype, freq_dtype=fdt, ratio=ratio, rotary_dim=rd, eps=1e-6, page_pad=pad)
    announce("compress %s/%s d=%d ratio=%d rd=%d page=%d pad=%d" % (dtype, fdt, d, ratio, rd, ps, pad))
    got = run(case)
    check(got, oracle.run_case(case), dtype, "compress %s d=%d ratio=%d" % (dtype, d, ratio))


def test_compress_max_blocks_cap_and_eps():
    """max_blocks below some sequences' block counts (those are cut at the stride), and
    a large eps that the norm must add."""
    case = W.make_compress(name="compress_cap", seed=62, cache_lengths=[300, 20, 90], rows=[1, 1, 1],
                           page_size=16, num_layers=1, layer_idx=0, head_dim=128, dtype="bf16", ratio=4,
                           rotary_dim=64, eps=0.75, max_blocks=40, std=0.5)
    announce("compress max_blocks cap")
    check(run(case), oracle.run_case(case), "bf16", "compress cap")


def test_compress_launch_bound_from_length_hints():
    """Blocks past (max_cache_length + max_prompt_length) / ratio are not computed: with
    the hints at 100 + 1 keys, sequence 0 (301 keys) gets 25 block keys and its later
    rows keep the canary; the other sequences are complete."""
    case = W.make_compress(name="compress_hint", seed=63, cache_lengths=[300, 20, 90], rows=[1, 1, 1],
                           page_size=16, num_layers=1, layer_idx=0, head_dim=64, dtype="f32", ratio=4,
                           rotary_dim=64)
    announce("compress launch bound from hints")
    got = run(case, kv_override={"max_cache_length": 100}, mpl=1)
    ref = oracle.run_case(case)
    ref = ref.reshape(case.batch, case.max_blocks, -1).copy()
    ref[:, 101 // 4:] = np.nan
    check(got, ref.reshape(case.batch * case.max_blocks, -1), "f32", "compress hint bound")


def test_compress_never_reads_past_complete_groups():
    """NaN at every raw position at or past each sequence's last complete group: the
    block keys are unchanged and finite."""
    case = W.make_compress(name="compress_nan", seed=64, cache_lengths=[13, 30, 5, 7, 129], rows=[3, 1, 2, 1, 1],
                           page_size=8, num_layers=2, layer_idx=1, head_dim=128, dtype="bf16", ratio=4,
                           rotary_dim=64)
    clean = oracle.run_case(case)
    c2 = copy.copy(case)
    c2.kv = copy.copy(case.kv)
    c2.kv.storage = case.kv.storage.clone()
    pv = c2.kv.pages_view()
    for b, nb in enumerate(case.blocks_per_sequence()):
        for p in range(int(nb) * case.ratio, case.kv.max_pages * case.kv.page_size):
            pv[int(c2.kv.lookup_table[b, p // case.kv.page_size]), 0, case.layer_idx, p % case.kv.page_size] = \
                float("nan")
    announce("compress NaN past complete groups")
    check(run(c2), clean, "bf16", "compress poisoned tail")


def test_compress_page_outside_pool_drops_its_blocks():
    """A page-table entry naming a page outside the pool: the blocks with a raw key in
    that logical page are not written; every other block key is exact."""
    case = W.make_compress(name="compress_badpage", seed=65, cache_lengths=[200, 90], rows=[1, 1], page_size=16,
                           num_layers=1, layer_idx=0, head_dim=128, dtype="bf16", ratio=4, rotary_dim=64)
    ref = oracle.run_case(case)
    c2 = copy.copy(case)
    c2.kv = copy.copy(case.kv)
    c2.kv.lookup_table = case.kv.lookup_table.copy()
    c2.kv.lookup_table[0, 3] = case.kv.num_pages + 5          # positions 48..63 of sequence 0
    ref = ref.reshape(2, case.max_blocks, -1).copy()
    ref[0, 48 // 4:64 // 4] = np.nan
    announce("compress page outside the pool")
    check(run(c2), ref.reshape(2 * case.max_blocks, -1), "bf16", "compress bad page")


def test_compress_full_size_indexer_workload():
    """The indexer key-compression workload at full size (32 sequences of 16k-32k raw
    keys, D 128 bf16, ratio 4, 64 rotary channels): every block key."""
    announce("compress full size: generating")
    case = W.f2_compress_keys_bf16()
    ref = oracle.run_case(case)
    announce("compress full size: running")
    err = check(run(case), ref, "bf16", "compress full size")
    announce("compress full size: max abs err %.3e" % err)


def test_compress_repeat_is_bitwise_identical():
    case = W.make_compress(name="compress_rep", seed=66, cache_lengths=[500, 77], rows=[1, 4], page_size=32,
                           num_layers=1, layer_idx=0, head_dim=128, dtype="bf16", ratio=4, rotary_dim=64)
    announce("compress repeat")
    assert torch.equal(run(case), run(case))


def test_compress_graph_replays_match_eager():
    """Captured in a HIP graph (no workspace, no memset): every replay, with eager work
    in between, reproduces the eager call bit for bit."""
    case = W.make_compress(name="compress_graph", seed=67, cache_lengths=[700, 50, 301], rows=[1, 2, 1],
                           page_size=64, num_layers=2, layer_idx=1, head_dim=128, dtype="bf16", ratio=4,
                           rotary_dim=64)
    dc = D.compress_to_device(case, DEV)
    out = torch.full((case.batch * case.max_blocks, case.head_dim), CANARY, dtype=torch.bfloat16, device=DEV)
    announce("compress graph: eager")
    eager = D.run_compress(dc, out=out).clone()
    torch.cuda.synchronize()
    check(eager, oracle.run_case(case), "bf16", "compress graph eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            D.run_compress(dc, out=out, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(4):
        announce("compress graph: replay %d" % k)
        out.fill_(CANARY)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager call" % k
    del g
