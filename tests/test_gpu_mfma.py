"""GPU parity of the matrix-core path (groups of 8 and 16 query heads per kv head):
index-selected prefill rows (bf16, group 16, the ragged-prefill workload's shape) and
block-sparse top-k decode (e4m3 and bf16, group 8), against the fp64 oracle."""
import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(case, options=None, rows=None):
    dc = D.to_device(case, DEV)
    out = D.run(dc, options=options)
    torch.cuda.synchronize()
    ref = oracle.run_case(case, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    return got, ref, out


def prefill_small(seed=3, rows=(40, 7, 70), cache=(300, 0, 900), g=16, d=128, W_=256, hkv=2, out="bf16",
                  dtype="bf16"):
    return W.make_qsa(name="prefill_small", seed=seed, rows=list(rows), cache_lengths=list(cache),
                      page_size=128, num_layers=1, layer_idx=0, num_kv_heads=hkv, group=g, head_dim=d,
                      dtype=dtype, out_dtype=out, selection_width=W_, selection="recent", recent=64,
                      scale=1 / np.sqrt(d))


@pytest.mark.parametrize("g,d,out", [(16, 128, "bf16"), (16, 128, "f32"), (8, 128, "f32"), (16, 64, "f32"),
                                     (12, 256, "f32"), (12, 64, "bf16"), (8, 256, "bf16")])
def test_qsa_mfma_shapes(g, d, out):
    case = prefill_small(g=g, d=d, out=out)
    announce("qsa mfma g=%d d=%d out=%s" % (g, d, out))
    got, ref, _ = run(case)
    # tolerance of the input type (bf16): P is rounded to bf16 for the P.V product
    compare(got, ref, "bf16", "mfma g=%d d=%d" % (g, d))


@pytest.mark.parametrize("splits,waves", [(1, 1), (1, 4), (3, 2), (8, 4)])
def test_qsa_mfma_splits_and_waves(splits, waves):
    case = prefill_small(seed=5, rows=(9, 3), cache=(500, 1200), W_=400, out="f32")
    announce("qsa mfma splits=%d waves=%d" % (splits, waves))
    got, ref, _ = run(case, options={"num_splits": splits, "waves": waves})
    compare(got, ref, "bf16", "mfma splits=%d waves=%d" % (splits, waves))


def test_qsa_mfma_e4m3_and_edges():
    case = prefill_small(seed=7, rows=(5, 0, 6), cache=(100, 3, 40), W_=48, dtype="e4m3", out="f32")
    c = copy.copy(case)
    c.counts = case.counts.copy()
    c.counts[0] = 0
    c.counts[1] = 1
    announce("qsa mfma e4m3 edges")
    got, ref, _ = run(c)
    assert (to64(got[0]) == 0).all()
    compare(got, ref, "e4m3", "mfma e4m3 edges")


def test_qsa_mfma_counts_one_exact():
    case = prefill_small(seed=9, rows=(4, 3), cache=(50, 200), W_=32, out="bf16")
    c = copy.copy(case)
    c.counts = np.ones_like(case.counts)
    announce("qsa mfma counts=1")
    dc = D.to_device(c, DEV)
    out = D.run(dc)
    torch.cuda.synchronize()
    pv = case.kv.pages_view()
    G = case.num_q_heads // case.kv.num_kv_heads
    pos = case.positions()
    off = case.input_row_offsets
    for r in range(case.total_q):
        b = int(np.searchsorted(off, r, side="right") - 1)
        p = int(case.token_indices[r, 0])
        page = int(case.kv.lookup_table[b, p // case.kv.page_size])
        v = pv[page, 1, 0, p % case.kv.page_size].repeat_interleave(G, dim=0)
        assert torch.equal(out[r].cpu().view(torch.int16), v.view(torch.int16)), (r, pos[r])


def test_qsa_mfma_e4m3_values_exact_every_code():
    """counts = 1 on the e4m3 matrix-core path returns the selected V row exactly, with
    the V rows holding every finite e4m3 code between them: pins the kernel's e4m3 ->
    bf16 widening of V (byte order and exactness) against torch's e4m3 decoding."""
    case = prefill_small(seed=13, rows=(3, 2), cache=(40, 90), W_=16, g=8, d=128, dtype="e4m3", out="bf16")
    c = copy.copy(case)
    c.counts = np.ones_like(case.counts)
    pv = case.kv.pages_view().view(torch.uint8)
    H, ps = case.kv.num_kv_heads, case.kv.page_size
    off = case.input_row_offsets
    sel = []
    for r in range(case.total_q):
        b = int(np.searchsorted(off, r, side="right") - 1)
        p = int(case.token_indices[r, 0])
        sel.append((int(case.kv.lookup_table[b, p // ps]), p % ps))
    # V rows of the selected keys, kv head g: codes (k * 128 + d) mod 256, the two NaN
    # codes replaced by zero (distinct selections first, so every code appears)
    distinct = sorted(set(sel))
    assert len(distinct) * H * 128 >= 256
    for k, (page, slot) in enumerate(distinct):
        for g in range(H):
            codes = (np.arange(128) + (k * H + g) * 128) % 256
            codes[(codes == 0x7F) | (codes == 0xFF)] = 0
            pv[page, 1, 0, slot, g] = torch.from_numpy(codes.astype(np.uint8))
    announce("qsa mfma e4m3 counts=1, every finite code")
    dc = D.to_device(c, DEV)
    out = D.run(dc)
    torch.cuda.synchronize()
    G = case.num_q_heads // H
    seen = set()
    for r, (page, slot) in enumerate(sel):
        raw = pv[page, 1, 0, slot]                                   # [H, D] codes
        v = raw.view(torch.float8_e4m3fn).float().repeat_interleave(G, dim=0)
        assert torch.equal(out[r].cpu().float(), v), r
        seen.update(raw.flatten().tolist())
    assert seen == set(range(256)) - {0x7F, 0xFF}


def test_c3_prefill_full_size_all_rows():
    """The ragged-prefill workload at full size (8 sequences, ~9.7k rows, group 16) in
    the default launch configuration; the oracle checks every row."""
    announce("c3 full size: generating")
    case = W.c3_prefill_bf16()
    announce("c3 full size: running (%d rows, all checked)" % case.total_q)
    got, ref, _ = run(case)
    compare(got, ref, "bf16", "c3 full")


# ----------------------------------------------------------------- block-sparse

def block_small(seed=21, dtype="e4m3", rows=None, cache=(900, 2000, 300), topk=5, g=8, hkv=2):
    return W.make_block_sparse(name="bs_small", seed=seed, cache_lengths=list(cache), rows=rows,
                               page_size=128, num_kv_heads=hkv, group=g, head_dim=128, dtype=dtype,
                               topk=topk, block_size=64, scale=1 / np.sqrt(128), std=0.5)


@pytest.mark.parametrize("dtype,g", [("e4m3", 8), ("bf16", 8), ("bf16", 16), ("e4m3", 4), ("bf16", 2)])
def test_block_sparse_small(dtype, g):
    case = block_small(dtype=dtype, g=g)
    announce("block-sparse %s g=%d" % (dtype, g))
    got, ref, _ = run(case)
    compare(got, ref, dtype, "block-sparse %s g=%d" % (dtype, g))


def test_block_sparse_prefill_rows_and_splits():
    case = block_small(seed=22, rows=[3, 1, 2], topk=4)
    for splits in (1, 2, 4):
        announce("block-sparse prefill rows splits=%d" % splits)
        got, ref, _ = run(case, options={"num_splits": splits})
        compare(got, ref, "e4m3", "block-sparse splits=%d" % splits)


def test_block_sparse_speculative_decode_full_size():
    """Speculative decode at the C4 shapes: 32 sequences x 3 draft tokens, each token at
    its own position with its own top-16 blocks and causal clip (the pages route 2-4
    query tokens per sequence to a separate kernel; here the one gather kernel takes
    every row's position from its sequence's cache length and its index). All rows."""
    announce("block-sparse spec decode: generating")
    case = W.c4s_block_sparse_spec_fp8()
    announce("block-sparse spec decode: running (%d rows)" % case.total_q)
    got, ref, _ = run(case)
    compare(got, ref, "e4m3", "block-sparse spec decode")


def test_block_sparse_prefill_all_rows():
    """Block-sparse prefill: 4 sequences x 96 new tokens, bf16, every row."""
    case = W.c4p_block_sparse_prefill_bf16()
    announce("block-sparse prefill: running (%d rows)" % case.total_q)
    got, ref, _ = run(case)
    compare(got, ref, "bf16", "block-sparse prefill")


def test_block_sparse_clip_never_reads_past_position():
    """Slots after a row's position in its last block hold NaN in the cache; the
    causal clip must keep them out of the result."""
    case = block_small(seed=23, cache=(64 * 7 + 5, 64 * 5 + 63, 64 * 9))
    announce("block-sparse clip")
    got, ref, _ = run(case)
    compare(got, ref, "e4m3", "block-sparse clip")


def test_c4_block_sparse_full_size():
    announce("c4 full size: generating")
    case = W.c4_block_sparse_fp8()
    announce("c4 full size: running")
    got, ref, _ = run(case)
    mx, rel = compare(got, ref, "e4m3", "c4 full")
    announce("c4 max abs %.3e rel-rms %.3e" % (mx, rel))


def test_shared_workspace_across_plans_and_shapes():
    """One workspace passed to split-K calls of different kernels, split counts and
    shapes in a row (wavefront and matrix-core kernels, larger and smaller shapes):
    nothing a call leaves in it changes a later call's result."""
    cases = [
        (block_small(seed=61, dtype="e4m3", cache=(900, 2000, 300, 4000)), {"num_splits": 4}),
        (W.make_qsa(name="ws_valu", seed=62, rows=[1] * 5, cache_lengths=[300, 900, 1200, 40, 700], page_size=128,
                    num_layers=1, layer_idx=0, num_kv_heads=2, group=4, head_dim=128, dtype="bf16",
                    out_dtype="bf16", selection_width=512, selection="uniform_counts", scale=1 / np.sqrt(128)),
         {"num_splits": 3}),
        (block_small(seed=63, dtype="e4m3", rows=[2, 1, 3], cache=(700, 3000, 500), topk=6), {"num_splits": 7}),
        (block_small(seed=64, dtype="e4m3", cache=(500, 260)), {"num_splits": 2}),
        (prefill_small(seed=65, rows=(12, 5), cache=(400, 900), g=16, d=64, out="f32"), {"num_splits": 5}),
        (block_small(seed=66, dtype="e4m3", cache=(900, 2000, 300, 4000)), {"num_splits": 4}),
    ]
    dcs = [(D.to_device(c, DEV), o) for c, o in cases]
    ws = torch.full((max(D.workspace_size(dc, o) for dc, o in dcs),), 255, dtype=torch.uint8, device=DEV)
    for k, ((case, _), (dc, opts)) in enumerate(zip(cases, dcs)):
        announce("shared workspace call %d (%s, %s)" % (k, case.kind, opts))
        out = D.run(dc, options=opts, workspace=ws)
        torch.cuda.synchronize()
        compare(out, oracle.run_case(case), "e4m3" if case.dtype == "e4m3" else
                ("f32" if case.out_dtype == "f32" and case.dtype == "f32" else "bf16"), "shared workspace %d" % k)
