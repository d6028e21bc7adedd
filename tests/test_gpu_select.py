"""GPU parity of top-k block selection (block keys -> token_indices, counts, block ids)
against the fp64 oracle.

With whole-number queries and keys in [-2, 2] every score is exact in fp32 whatever the
order of the sums, so the kernel and the oracle take the same decisions, ties included
(equal scores go to the lower block index): those cases compare token indices, counts
and block ids exactly. With continuous values, blocks whose scores differ by less than
fp32 rounding may be chosen either way, so those cases check what is unique (counts,
the incomplete group, increasing order, the block count) and that the kept set is a
valid top-k of the fp64 scores: no dropped block outscores a kept one by more than
1e-3. Entries past a row's count must keep the caller's values. Also covered: every
team width, ratios 1 to 16, topk 0, rows before their first complete group, more
candidates than topk and fewer, the large-candidate path (over 4096 blocks), the
full-size indexer selection, and the chain key compression -> selection -> sparse
attention through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
FILL = -7


def run(case):
    dc = D.select_to_device(case, DEV)
    idx = torch.full((case.total_q, case.W), FILL, dtype=torch.int32, device=DEV)
    counts = torch.full((case.total_q,), FILL, dtype=torch.int32, device=DEV)
    blocks = torch.full((case.total_q, case.topk), FILL, dtype=torch.int32, device=DEV) if case.topk else None
    D.run_select(dc, token_indices=idx, counts=counts, blocks=blocks)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), counts.cpu().numpy(), blocks.cpu().numpy() if blocks is not None else None)


def check_exact(case, got, what):
    ref = oracle.run_case(case)
    idx, counts, blocks = got
    assert np.array_equal(counts, ref[1]), what + ": counts differ"
    for r in range(case.total_q):
        n = ref[1][r]
        assert np.array_equal(idx[r, :n], ref[0][r, :n]), "%s row %d: token indices differ" % (what, r)
        assert (idx[r, n:] == FILL).all(), "%s row %d: wrote past the count" % (what, r)
    if case.topk:
        assert np.array_equal(blocks, ref[2]), what + ": block ids differ"


def scores64(case):
    q = case.q_index.float().double().numpy()
    bk = case.block_keys.float().double().numpy().reshape(case.batch, case.max_blocks, -1)
    return q, bk


def check_valid(case, got, what, eps=1e-3):
    idx, counts, blocks = got
    ref = oracle.run_case(case)
    q, bk = scores64(case)
    off = case.input_row_offsets.astype(np.int64)
    pos = case.positions()
    assert np.array_equal(counts, ref[1]), what + ": counts differ"
    for r in range(case.total_q):
        b = int(np.searchsorted(off, r, side="right") - 1)
        nfull = (pos[r] + 1) // case.ratio
        nv = min(nfull, case.max_blocks)
        k = min(case.topk, nv)
        kept = blocks[r, :k]
        assert (blocks[r, k:] == -1).all() and (np.diff(kept) > 0).all() and (kept >= 0).all() and \
            (kept < nv).all(), "%s row %d: block ids %s" % (what, r, blocks[r].tolist())
        toks = [int(j) * case.ratio + t for j in kept for t in range(case.ratio)] + \
            list(range(nfull * case.ratio, pos[r] + 1))
        assert idx[r, :counts[r]].tolist() == toks, "%s row %d: token indices do not match the block ids" % (what, r)
        assert (idx[r, counts[r]:] == FILL).all(), "%s row %d: wrote past the count" % (what, r)
        if 0 < k < nv:
            s = bk[b, :nv] @ q[r]
            mask = np.zeros(nv, bool)
            mask[kept] = True
            assert s[mask].min() >= s[~mask].max() - eps, "%s row %d: not a top-%d (%.6f < %.6f)" % (
                what, r, k, s[mask].min(), s[~mask].max())


EXACT = [
    # dtype, head_dim, ratio, topk, rows, cache lengths
    ("bf16", 128, 4, 5, [1, 3, 2, 1], [40, 23, 2, 77]),
    ("f32", 64, 3, 7, [2, 1, 4], [100, 9, 60]),
    ("bf16", 16, 1, 4, [3, 1], [12, 0]),
    ("bf16", 512, 16, 2, [1, 2], [500, 33]),
    ("f32", 256, 4, 0, [2, 1], [30, 5]),
    ("bf16", 8, 2, 64, [1, 1, 1], [300, 90, 1]),
    ("bf16", 128, 4, 300, [1, 1, 2], [4000, 1000, 20]),
    ("bf16", 128, 4, 100, [1, 2], [20000, 17000]),          # over 4096 candidates
    ("bf16", 64, 1, 5000, [1, 2], [9000, 6000]),            # more kept blocks than LDS stages
    ("f32", 32, 2, 4096, [1, 1], [8200, 3000]),             # exactly as many as it stages
    ("bf16", 128, 4, 2000, [1], [6000]),                    # every candidate kept, over 1024
    ("f32", 256, 2, 9, [2, 1], [300, 77]),                  # 1024-byte key rows: 64-lane teams
]


@pytest.mark.parametrize("dtype,d,ratio,topk,rows,cl", EXACT)
def test_select_exact_on_whole_numbers(dtype, d, ratio, topk, rows, cl):
    case = W.make_select(name="sel_t", seed=71, rows=rows, cache_lengths=cl, head_dim=d, dtype=dtype, ratio=ratio,
                         topk=topk, integer=True)
    announce("select exact %s d=%d ratio=%d topk=%d max_blocks=%d" % (dtype, d, ratio, topk, case.max_blocks))
    check_exact(case, run(case), "select %s d=%d ratio=%d topk=%d" % (dtype, d, ratio, topk))


@pytest.mark.parametrize("dtype,d,ratio,topk,rows,cl", [
    ("bf16", 128, 4, 64, [1, 4, 1], [3000, 700, 90]),
    ("f32", 128, 8, 16, [2, 2], [2000, 400]),
    ("bf16", 128, 4, 511, [1, 1], [30000, 9000]),
])
def test_select_valid_on_continuous_values(dtype, d, ratio, topk, rows, cl):
    case = W.make_select(name="sel_c", seed=72, rows=rows, cache_lengths=cl, head_dim=d, dtype=dtype, ratio=ratio,
                         topk=topk)
    announce("select continuous %s d=%d ratio=%d topk=%d" % (dtype, d, ratio, topk))
    check_valid(case, run(case), "select continuous %s" % dtype)


def test_select_max_blocks_cap():
    case = W.make_select(name="sel_cap", seed=73, rows=[1, 2], cache_lengths=[90, 200], head_dim=64, dtype="bf16",
                         ratio=4, topk=6, max_blocks=20, integer=True)
    announce("select max_blocks cap")
    check_exact(case, run(case), "select cap")


def test_select_without_max_cache_length():
    """max_cache_length 0 (no hint): every complete block is still a candidate, and the
    result equals the oracle's and the call with the hint."""
    import sparse_attention_ragged_amd as qsa
    case = W.make_select(name="sel_nohint", seed=74, rows=[1, 3, 2], cache_lengths=[300, 1200, 40], head_dim=128,
                         dtype="bf16", ratio=4, topk=16, integer=True)
    dc = D.select_to_device(case, DEV)
    outs = []
    for mcl in (0, int(np.max(case.cache_lengths))):
        announce("select max_cache_length=%d" % mcl)
        idx = torch.full((case.total_q, case.W), FILL, dtype=torch.int32, device=DEV)
        counts = torch.full((case.total_q,), FILL, dtype=torch.int32, device=DEV)
        blocks = torch.full((case.total_q, case.topk), FILL, dtype=torch.int32, device=DEV)
        qsa.select_blocks(dc.q_index, dc.row_off, dc.block_keys, dc.cache_lengths, case.max_blocks, case.ratio,
                          case.topk, selection_width=case.W, max_cache_length=mcl,
                          max_prompt_length=case.max_prompt_length, token_indices=idx, counts=counts, blocks=blocks)
        torch.cuda.synchronize()
        got = (idx.cpu().numpy(), counts.cpu().numpy(), blocks.cpu().numpy())
        check_exact(case, got, "select max_cache_length=%d" % mcl)
        outs.append(got)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_select_full_size_indexer_workload():
    """Selection at the indexer workload's shapes (32 rows, 4k-8k candidate blocks of 4
    positions, top 511 blocks into 2047 positions)."""
    announce("select full size: generating")
    case = W.f4_select_blocks_bf16()
    announce("select full size: running")
    check_valid(case, run(case), "select full size")


def test_chain_compress_select_attend():
    """Key compression, block selection and sparse attention through the C ABI, each
    checked against the oracle on the previous step's GPU output."""
    import sparse_attention_ragged_amd as qsa
    comp = W.make_compress(name="chain", seed=74, cache_lengths=[700, 301, 1200], rows=[1, 1, 1], page_size=64,
                           num_layers=1, layer_idx=0, head_dim=128, dtype="bf16", ratio=4, rotary_dim=64)
    dcomp = D.compress_to_device(comp, DEV)
    announce("chain: compress")
    bk = torch.zeros((comp.batch * comp.max_blocks, 128), dtype=torch.bfloat16, device=DEV)
    D.run_compress(dcomp, out=bk)
    torch.cuda.synchronize()
    ref_bk = oracle.run_case(comp)
    live = ~np.isnan(ref_bk).all(axis=1)
    got_bk = bk.float().cpu().double().numpy()
    assert (np.abs(got_bk[live] - ref_bk[live]) <= np.maximum(2e-2, np.abs(ref_bk[live]) / 256)).all()
    # selection over the GPU block keys: one decode row per sequence at its last position
    sel = W.make_select(name="chain_sel", seed=75, rows=[1, 1, 1], cache_lengths=[700, 301, 1200], head_dim=128,
                        dtype="bf16", ratio=4, topk=40, max_blocks=comp.max_blocks)
    sel.block_keys = bk.cpu()
    announce("chain: select")
    got = run(sel)
    check_valid(sel, got, "chain select")
    # attention over the selected positions (a K/V cache of the same sequences)
    att = W.make_qsa(name="chain_att", seed=76, rows=[1, 1, 1], cache_lengths=[700, 301, 1200], page_size=64,
                     num_layers=1, layer_idx=0, num_kv_heads=2, group=4, head_dim=128, dtype="bf16", out_dtype="bf16",
                     selection_width=sel.W, selection="min", scale=1 / np.sqrt(128))
    att.token_indices = got[0].copy()
    att.counts = got[1].copy()
    announce("chain: attend")
    datt = D.to_device(att, DEV)
    out = D.run(datt)
    torch.cuda.synchronize()
    compare(out, oracle.run_case(att), "bf16", "chain attention")


def test_select_graph_replays_match_eager():
    """Captured in a HIP graph with a caller-provided workspace (no allocation, no
    memset): every replay, with eager work in between, reproduces the eager call."""
    import sparse_attention_ragged_amd as qsa
    case = W.make_select(name="sel_graph", seed=77, rows=[1, 3, 2], cache_lengths=[900, 300, 5000], head_dim=128,
                         dtype="bf16", ratio=4, topk=50, integer=True)
    dc = D.select_to_device(case, DEV)
    n = qsa.select_blocks_workspace_size(dc.q_index, dc.row_off, case.max_blocks, case.ratio, case.topk,
                                         int(np.max(case.cache_lengths)), case.max_prompt_length)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    idx = torch.full((case.total_q, case.W), FILL, dtype=torch.int32, device=DEV)
    counts = torch.zeros(case.total_q, dtype=torch.int32, device=DEV)
    blocks = torch.zeros((case.total_q, case.topk), dtype=torch.int32, device=DEV)
    announce("select graph: eager")
    D.run_select(dc, token_indices=idx, counts=counts, blocks=blocks, workspace=ws)
    torch.cuda.synchronize()
    eager = (idx.clone(), counts.clone(), blocks.clone())
    check_exact(case, (eager[0].cpu().numpy(), eager[1].cpu().numpy(), eager[2].cpu().numpy()), "select graph eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            D.run_select(dc, token_indices=idx, counts=counts, blocks=blocks, workspace=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(4):
        announce("select graph: replay %d" % k)
        idx.fill_(FILL)
        counts.zero_()
        blocks.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, eager[0]) and torch.equal(counts, eager[1]) and torch.equal(blocks, eager[2]), \
            "replay %d differs from the eager call" % k
    del g
