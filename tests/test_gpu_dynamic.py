"""GPU parity of the dynamically scheduled wavefront kernel (persistent workgroups take
key-range units from a counter; a combine step merges the units' partials) against
the fp64 oracle: every element type and group of the wavefront path, all three key
lists, ragged and zero counts (units past a row's length are skipped), fewer units than
workgroups, the full-size decode workload against both the oracle and the statically
scheduled kernel, and repeated calls on one workspace (the work counter is back at zero
after each call)."""
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
DYN = {"schedule": "dynamic"}
STATIC = {"schedule": "static"}


def decode(seed, batch, lo, hi, W_, g=4, d=128, dtype="bf16", out="bf16", hkv=8, sel="uniform_counts"):
    rng = np.random.default_rng(seed + 5000)
    cl = rng.integers(lo, hi, size=batch, endpoint=True)
    return W.make_qsa(name="decode_dyn", seed=seed, rows=[1] * batch, cache_lengths=cl, page_size=128,
                      num_layers=2, layer_idx=1, num_kv_heads=hkv, group=g, head_dim=d, dtype=dtype,
                      out_dtype=out, selection_width=W_, selection=sel, scale=1 / np.sqrt(d))


def run(case, options, rows=None, workspace=None):
    dc = D.to_device(case, DEV)
    out = D.run(dc, options=options, workspace=workspace)
    torch.cuda.synchronize()
    ref = oracle.run_case(case, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    return got, ref, dc


@pytest.mark.parametrize("dtype,g,d,out", [("bf16", 4, 128, "bf16"), ("f32", 4, 64, "f32"), ("e4m3", 4, 128, "bf16"),
                                           ("bf16", 1, 64, "f32"), ("bf16", 2, 256, "bf16"), ("f32", 1, 128, "f32"),
                                           ("e4m3", 2, 256, "f32")])
def test_dynamic_matches_oracle(dtype, g, d, out):
    """Uniform counts in [1, min(W, pos + 1)]: most rows end inside their last units, and
    units past a row's length are written empty without being streamed."""
    case = decode(seed=71, batch=5, lo=50, hi=1500, W_=1200, g=g, d=d, dtype=dtype, out=out, hkv=4)
    announce("dynamic %s g=%d d=%d out=%s" % (dtype, g, d, out))
    got, ref, _ = run(case, DYN)
    compare(got, ref, dtype, "dynamic %s g=%d d=%d" % (dtype, g, d))


def test_dynamic_ragged_counts_full_width():
    """64 rows x 8 kv heads, W 2048, counts uniform in [1, min(W, pos + 1)]: about half of
    the units start past their row's length and are skipped, so streams end at
    different points of their slot rings. Regression case for the pipeline stages that
    run ahead of the fold: past a stream's empty end slot they must not read ring
    slots that were never published."""
    rng = np.random.default_rng(12)
    cl = rng.integers(2048, 8192, size=64, endpoint=True)
    case = W.make_qsa(name="decode_ragged", seed=12, rows=[1] * 64, cache_lengths=cl, page_size=128,
                      num_layers=4, layer_idx=2, num_kv_heads=8, group=4, head_dim=128, dtype="bf16",
                      out_dtype="bf16", selection_width=2048, selection="uniform_counts",
                      scale=1 / np.sqrt(128))
    announce("dynamic ragged counts, W 2048")
    got, ref, dc = run(case, DYN)
    compare(got, ref, "bf16", "dynamic ragged", rel_rms_max=0.01)
    sta = D.run(dc, options=STATIC)
    torch.cuda.synchronize()
    compare(sta, ref, "bf16", "static ragged", rel_rms_max=0.01)


def test_dynamic_zero_and_clamped_counts():
    case = decode(seed=72, batch=6, lo=600, hi=900, W_=512, hkv=2)
    c = copy.copy(case)
    c.counts = case.counts.copy()
    c.counts[0] = 0
    c.counts[3] = -4
    c.counts[5] = 10_000        # clamps to the width (the selection holds W entries)
    c.token_indices = case.token_indices.copy()
    pos5 = int(c.positions()[5])
    c.token_indices[5] = np.sort(np.random.default_rng(2).choice(pos5 + 1, 512, replace=False))
    announce("dynamic zero / negative / clamped counts")
    got, ref, _ = run(c, DYN)
    assert (to64(got[0]) == 0).all() and (to64(got[3]) == 0).all()
    compare(got, ref, "bf16", "dynamic counts edges")


def test_dynamic_all_rows_empty():
    case = decode(seed=73, batch=4, lo=100, hi=300, W_=256, hkv=2)
    c = copy.copy(case)
    c.counts = np.zeros_like(case.counts)
    announce("dynamic all rows empty")
    got, ref, _ = run(c, DYN)
    assert (to64(got) == 0).all()
    compare(got, ref, "bf16", "dynamic empty")


def test_dynamic_fewer_units_than_workgroups():
    case = W.c1_tiny_fp32()
    announce("dynamic c1 tiny (fewer units than workgroups)")
    got, ref, _ = run(case, DYN)
    compare(got, ref, "f32", "dynamic c1")


@pytest.mark.parametrize("dtype,g", [("e4m3", 4), ("bf16", 2), ("bf16", 1)])
def test_dynamic_block_sparse(dtype, g):
    case = W.make_block_sparse(name="bs_dyn", seed=74, cache_lengths=[900, 2000, 300, 4100], rows=[1, 3, 1, 2],
                               page_size=128, num_kv_heads=2, group=g, head_dim=128, dtype=dtype, topk=5,
                               block_size=64, scale=1 / np.sqrt(128), std=0.5)
    announce("dynamic block-sparse %s g=%d" % (dtype, g))
    got, ref, _ = run(case, DYN)
    compare(got, ref, dtype, "dynamic block-sparse %s g=%d" % (dtype, g))


@pytest.mark.parametrize("heads,d", [(4, 128), (2, 256), (1, 64)])
def test_dynamic_latent(heads, d):
    case = W.make_latent(name="lat_dyn", seed=75, decode_positions=[300, 1000, 77], prefill_positions=[500],
                         prefill_rows=9, num_heads=heads, head_dim=d, dtype="bf16", out_dtype="f32", window=24,
                         swa_page_size=16, comp_page_size=32, num_comp=300, comp_ratio=4, unused_frac=0.1,
                         scale=1 / np.sqrt(d))
    announce("dynamic latent heads=%d d=%d" % (heads, d))
    got, ref, _ = run(case, DYN)
    compare(got, ref, "bf16", "dynamic latent h=%d d=%d" % (heads, d))


def test_dynamic_repeat_agrees_and_counter_returns_to_zero():
    """Repeated calls on one workspace: the combine step leaves the work counter at
    zero after each, and the results agree to rounding (a unit's keys are spread over
    4 or 3 wavefronts depending on which of a workgroup's two streams takes it, which
    changes the order of the fp32 sums; the static schedule is bitwise reproducible)."""
    case = decode(seed=76, batch=40, lo=600, hi=3000, W_=1536, hkv=8, sel="min")
    dc = D.to_device(case, DEV)
    n = D.workspace_size(dc, DYN)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref = oracle.run_case(case)
    for k in range(3):
        announce("dynamic repeat %d" % k)
        out = D.run(dc, options=DYN, workspace=ws)
        torch.cuda.synchronize()
        counter = ws[n - 256:n - 252].view(torch.int32).item()
        assert counter == 0, "work counter left at %d" % counter
        compare(out, ref, "bf16", "dynamic repeat %d" % k, rel_rms_max=0.01)


def test_static_schedule_is_bitwise_reproducible():
    case = decode(seed=77, batch=40, lo=600, hi=3000, W_=1536, hkv=8, sel="min")
    dc = D.to_device(case, DEV)
    announce("static repeat")
    a = D.run(dc, options=STATIC)
    b = D.run(dc, options=STATIC)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dynamic_c2_full_size_matches_oracle_and_static():
    """The bf16 decode workload at full size (64 rows x 8 kv heads, W 2048): the
    dynamic schedule against the oracle on every row, and against the statically
    scheduled kernel (the automatic choice)."""
    announce("c2 dynamic: generating")
    case = W.c2_decode_bf16()
    dc = D.to_device(case, DEV)
    ref = oracle.run_case(case)
    announce("c2 dynamic: running")
    auto = D.run(dc)
    dyn = D.run(dc, options=DYN)
    sta = D.run(dc, options=STATIC)
    torch.cuda.synchronize()
    # the automatic plan is the static one (same workspace layout)
    assert D.workspace_size(dc, None) == D.workspace_size(dc, STATIC) != D.workspace_size(dc, DYN)
    compare(auto, ref, "bf16", "c2 auto", rel_rms_max=0.01)
    compare(dyn, ref, "bf16", "c2 dynamic", rel_rms_max=0.01)
    compare(sta, ref, "bf16", "c2 static", rel_rms_max=0.01)
    # both round to bf16 from fp32 sums that differ in order and in where P is rounded
    assert np.abs(to64(dyn) - to64(sta)).max() <= 2e-2
