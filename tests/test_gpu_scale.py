"""GPU parity at non-positive softmax scales against the fp64 oracle. The matrix-core
kernels apply a positive scale once to the running maximum and fold it into the
exponent's FMA; any other finite scale (negative: the softmax favours the smallest
scores; zero: every present key weighs the same) takes the plain path that scales
each score first. Both paths must give the oracle's result on every kernel family:
wavefront (groups up to 4), key-split matrix core (bf16 group 16, e4m3 group 8), the
dense shared-tile kernel, and the head-split latent kernel."""
import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALES = [-0.125, 0.0, 0.0625]


def run(case):
    dc = D.to_device(case, DEV)
    out = D.run(dc)
    torch.cuda.synchronize()
    return out, oracle.run_case(case)


def with_scale(case, scale):
    c = copy.copy(case)
    c.scale = float(scale)
    return c


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("g,dtype", [(16, "bf16"), (8, "e4m3"), (4, "bf16")])
def test_selected_keys_any_scale(scale, g, dtype):
    case = W.make_qsa(name="scale_qsa", seed=91, rows=[20, 3, 33], cache_lengths=[400, 0, 700], page_size=64,
                      num_layers=1, layer_idx=0, num_kv_heads=2, group=g, head_dim=128, dtype=dtype, out_dtype="f32",
                      selection_width=200, selection="recent", recent=32, scale=0.1)
    case = with_scale(case, scale)
    announce("selected keys scale=%g g=%d %s" % (scale, g, dtype))
    got, ref = run(case)
    compare(got, ref, "bf16" if dtype == "bf16" else dtype, "scale %g g=%d" % (scale, g))


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("g", [16, 4])
def test_dense_any_scale(scale, g):
    case = W.make_dense(name="scale_dense", seed=92, rows=[70, 1, 129], num_kv_heads=2, group=g, head_dim=128,
                        dtype="bf16", out_dtype="f32", causal=True, window=-1, scale=0.1)
    case = with_scale(case, scale)
    announce("dense scale=%g g=%d" % (scale, g))
    got, ref = run(case)
    compare(got, ref, "bf16", "dense scale %g g=%d" % (scale, g))


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("heads,d", [(64, 512), (16, 128)])
def test_latent_any_scale(scale, heads, d):
    case = W.make_latent(name="scale_latent", seed=93, decode_positions=[300, 800], prefill_positions=[400],
                         prefill_rows=5, num_heads=heads, head_dim=d, dtype="bf16", out_dtype="f32", window=24,
                         swa_page_size=16, comp_page_size=32, num_comp=40, comp_ratio=4, unused_frac=0.1, scale=0.1)
    case = with_scale(case, scale)
    announce("latent scale=%g heads=%d" % (scale, heads))
    got, ref = run(case)
    compare(got, ref, "bf16", "latent scale %g heads=%d" % (scale, heads))
