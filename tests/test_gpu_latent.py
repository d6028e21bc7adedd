"""GPU parity of latent window + compressed + sink attention against the fp64 oracle,
over every kernel family it can run on (wavefront dot products for 1-4 heads, the
key-split matrix-core kernel for 8-16 heads, the head-split matrix-core kernel for
17-64 heads), plus the full-size latent workload on sampled rows."""
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


def latent_small(seed=31, heads=64, d=512, dtype="bf16", out="bf16", unused=0.1, num_comp=40, window=24,
                 dec=(300, 1000, 77), pre=(500,), pre_rows=9):
    return W.make_latent(name="lat_small", seed=seed, decode_positions=list(dec), prefill_positions=list(pre),
                         prefill_rows=pre_rows, num_heads=heads, head_dim=d, dtype=dtype, out_dtype=out,
                         window=window, swa_page_size=16, comp_page_size=32, num_comp=num_comp, comp_ratio=4,
                         unused_frac=unused, scale=1 / np.sqrt(d))


def run(case, options=None, rows=None):
    dc = D.to_device(case, DEV)
    out = D.run(dc, options=options)
    torch.cuda.synchronize()
    ref = oracle.run_case(case, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    return got, ref


@pytest.mark.parametrize("heads,d,out", [(64, 512, "bf16"), (64, 512, "f32"), (32, 256, "f32"), (48, 128, "f32"),
                                         (40, 256, "f32"), (20, 512, "bf16"), (17, 128, "f32"), (33, 128, "bf16"),
                                         (48, 256, "bf16"),
                                         (16, 128, "f32"), (8, 256, "bf16"), (4, 128, "f32"), (2, 64, "f32")])
def test_latent_shapes(heads, d, out):
    case = latent_small(heads=heads, d=d, out=out)
    announce("latent heads=%d d=%d out=%s" % (heads, d, out))
    got, ref = run(case)
    compare(got, ref, "bf16", "latent h=%d d=%d" % (heads, d))


@pytest.mark.parametrize("heads", [64, 16, 4])
@pytest.mark.parametrize("splits", [2, 5])
def test_latent_splits_apply_sink_once(heads, splits):
    case = latent_small(seed=33, heads=heads, d=128, out="f32", num_comp=60)
    announce("latent splits=%d heads=%d" % (splits, heads))
    got, ref = run(case, options={"num_splits": splits})
    compare(got, ref, "bf16", "latent splits=%d" % splits)


def test_latent_window_only_and_no_sink():
    case = latent_small(seed=34, heads=64, d=256, out="f32")
    c = copy.copy(case)
    c.comp_indices = np.full_like(case.comp_indices, -1)
    c.attn_sink = np.full_like(case.attn_sink, -np.inf)
    announce("latent window only, no sink")
    got, ref = run(c)
    compare(got, ref, "bf16", "latent window-only")


def test_latent_large_sink_dominates():
    """A sink far above every score drives the output toward zero without overflow."""
    case = latent_small(seed=35, heads=32, d=128, out="f32")
    c = copy.copy(case)
    c.attn_sink = np.full_like(case.attn_sink, 80.0)
    announce("latent large sink")
    got, ref = run(c)
    assert np.isfinite(to64(got)).all()
    compare(got, ref, "bf16", "latent large sink")


def test_c5_latent_full_size_all_rows():
    """The latent workload at full size (16 decode + 4 x 128 prefill rows, 64 heads,
    head_dim 512) in the default launch configuration (528 rows fill two rounds of 256
    CUs plus 16: those 16 run split, the others unsplit); the oracle checks every row."""
    announce("c5 full size: generating")
    case = W.c5_latent_bf16()
    announce("c5 full size: running (%d rows, all checked)" % case.total_q)
    got, ref = run(case)
    compare(got, ref, "bf16", "c5 full")


@pytest.mark.parametrize("n_decode,tail", [(258, 2), (300, 44), (256 + 64, 64), (256 + 65, 65)])
def test_latent_tail_rows_run_split(n_decode, tail):
    """More rows than 256 CUs with a short last round: the last total_q mod 256 rows
    (at most 64 of them) run split and are merged by the combine step, the rows before
    them unsplit; with a longer last round every row runs unsplit. Every row checked."""
    rng = np.random.default_rng(n_decode)
    pos = rng.integers(30, 400, size=n_decode)
    case = W.make_latent(name="lat_tail", seed=n_decode, decode_positions=pos, prefill_positions=[],
                         prefill_rows=0, num_heads=64, head_dim=128, dtype="bf16", out_dtype="bf16", window=24,
                         swa_page_size=16, comp_page_size=16, num_comp=40, comp_ratio=4, unused_frac=0.2,
                         scale=1 / np.sqrt(128))
    assert case.total_q % 256 == tail
    announce("latent tail rows: %d rows (tail %d)" % (case.total_q, tail))
    got, ref = run(case)
    compare(got, ref, "bf16", "latent tail %d" % tail)
