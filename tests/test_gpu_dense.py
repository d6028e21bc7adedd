"""GPU parity of dense ragged attention without a KV cache (the comparison row for the
sparse operations) against the fp64 oracle: the wavefront kernel (groups 1, 2, 4) and
the matrix-core kernel (groups 8, 16), every element type, causal, sliding-window and
unmasked attention, one-row and empty sequences, split-K partitions, and the C3-shape
dense prefill on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dense(seed, rows, hkv, g, d, dtype, out="f32", causal=True, window=-1):
    return W.make_dense(name="dense_t", seed=seed, rows=rows, num_kv_heads=hkv, group=g, head_dim=d, dtype=dtype,
                        out_dtype=out, causal=causal, window=window, scale=1 / np.sqrt(d))


def run(case, options=None, rows=None):
    dc = D.to_device(case, DEV)
    out = D.run(dc, options=options)
    torch.cuda.synchronize()
    ref = oracle.run_case(case, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    return got, ref, dc


SHAPES = [
    # (dtype, hkv, group, head_dim, causal, window)   wavefront kernel
    ("f32", 2, 4, 64, True, -1),
    ("bf16", 4, 1, 128, True, 37),
    ("bf16", 2, 2, 256, False, -1),
    ("e4m3", 2, 4, 128, True, 100),
    ("f32", 1, 1, 128, False, 20),
    # matrix-core kernel
    ("bf16", 2, 16, 128, True, -1),
    ("e4m3", 2, 8, 128, False, -1),
    ("bf16", 1, 8, 64, True, 50),
    ("bf16", 2, 16, 256, True, 200),
]


@pytest.mark.parametrize("dtype,hkv,g,d,causal,window", SHAPES)
def test_dense_matches_oracle(dtype, hkv, g, d, causal, window):
    case = dense(81, [130, 1, 0, 257, 64], hkv, g, d, dtype, causal=causal, window=window)
    announce("dense %s hkv=%d g=%d d=%d causal=%s window=%d" % (dtype, hkv, g, d, causal, window))
    got, ref, _ = run(case)
    compare(got, ref, dtype, "dense %s g=%d d=%d" % (dtype, g, d))


def test_dense_window_one_is_v_rows():
    """With a window of one every row sees only itself: its output is its own V row."""
    case = dense(82, [9, 4, 17], 2, 4, 64, "f32", causal=True, window=1)
    announce("dense window 1")
    got, _, dc = run(case)
    v = dc.v.float().repeat_interleave(4, dim=1)
    assert torch.equal(got.float(), v)


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_dense_splits(splits):
    case = dense(83, [300, 45, 512], 2, 4, 128, "bf16", causal=True)
    announce("dense splits=%d" % splits)
    got, ref, _ = run(case, options={"num_splits": splits})
    compare(got, ref, "bf16", "dense splits=%d" % splits)
    case16 = dense(84, [300, 45, 512], 1, 16, 128, "bf16", causal=False)
    got, ref, _ = run(case16, options={"num_splits": splits})
    compare(got, ref, "bf16", "dense g16 splits=%d" % splits)


def test_dense_prefill_c3_shapes_sampled_rows():
    """Dense causal prefill at the C3 shapes (8 sequences of 256-2048 rows, 64 q / 4 kv
    heads, D 128, bf16): sampled rows including every sequence's first and last."""
    case = W.f3_dense_prefill_bf16()
    off = case.input_row_offsets.astype(int)
    rows = sorted(set(np.linspace(0, case.total_q - 1, 40).astype(int).tolist()) | set(off[:-1].tolist())
                  | set((off[1:] - 1).tolist()))
    announce("dense prefill c3 shapes (%d rows checked)" % len(rows))
    got, ref, _ = run(case, rows=rows)
    compare(got, ref, "bf16", "dense prefill")


@pytest.mark.parametrize("causal,window", [(True, -1), (False, -1), (True, 3), (False, 2)])
def test_dense_shared_tiles_across_short_sequences(causal, window):
    """Matrix-core groups without a split run four consecutive rows per workgroup over
    their shared key tiles; with many short sequences a workgroup's rows straddle
    sequence boundaries (the union of their key ranges is still contiguous) and each row
    must mask the other sequences' keys."""
    case = dense(85, [1, 2, 3, 1, 5, 7, 0, 4, 33, 1, 6], 2, 16, 128, "bf16", causal=causal, window=window)
    announce("dense short sequences causal=%s window=%d" % (causal, window))
    got, ref, _ = run(case)
    compare(got, ref, "bf16", "dense short sequences")


def test_dense_per_row_kernel_matches_shared_tiles():
    """The per-row matrix-core kernel (taken when a wavefront count is requested) and the
    shared-tile kernel (the automatic choice) both match the oracle."""
    case = dense(86, [300, 45, 129], 2, 16, 128, "bf16", causal=True)
    announce("dense per-row vs shared tiles")
    got_auto, ref, dc = run(case)
    got_rows, _, _ = run(case, options={"waves": 4})
    compare(got_auto, ref, "bf16", "dense shared tiles")
    compare(got_rows, ref, "bf16", "dense per-row")


@pytest.mark.parametrize("g,d", [(16, 64), (12, 128), (16, 256)])
def test_dense_shared_tiles_bf16_output(g, d):
    """bf16 output rows of the shared-tile kernel at every head_dim it is built for, with
    a group that leaves head slots of the 16-wide operand unused (group 12)."""
    case = dense(87 + d, [150, 7, 64, 1, 90], 2, g, d, "bf16", out="bf16", causal=True)
    announce("dense shared tiles bf16 out g=%d d=%d" % (g, d))
    got, ref, _ = run(case)
    compare(got, ref, "bf16", "dense bf16 out g=%d d=%d" % (g, d))
