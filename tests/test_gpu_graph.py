"""The C-ABI calls inside a captured HIP graph (torch.cuda.CUDAGraph over the library's
launches on the capture stream): the library allocates nothing and records no memset,
so a captured call can be replayed.
Each graph is replayed several times with eager work and synchronisation in between,
and every replay is checked against the eager result of the same call."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import device as D
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def decode(seed=91, batch=24, lo=300, hi=2500, W_=1024, g=4, d=128, hkv=8):
    rng = np.random.default_rng(seed + 5000)
    cl = rng.integers(lo, hi, size=batch, endpoint=True)
    return W.make_qsa(name="decode_graph", seed=seed, rows=[1] * batch, cache_lengths=cl, page_size=128,
                      num_layers=2, layer_idx=1, num_kv_heads=hkv, group=g, head_dim=d, dtype="bf16",
                      out_dtype="bf16", selection_width=W_, selection="uniform_counts", scale=1 / np.sqrt(d))


CASES = {
    "one split": (lambda: decode(), {"num_splits": 1}),
    "split-K": (lambda: decode(), {"num_splits": 4}),
    "block-sparse split-K": (lambda: W.make_block_sparse(
        name="bs_graph", seed=92, cache_lengths=[900, 2000, 300, 4100], rows=[1, 3, 1, 2], page_size=128,
        num_kv_heads=2, group=8, head_dim=128, dtype="e4m3", topk=5, block_size=64, scale=1 / np.sqrt(128)),
        None),
    "dense": (lambda: W.make_dense(name="dense_graph", seed=93, rows=[130, 1, 257], num_kv_heads=2, group=4,
                                   head_dim=128, dtype="bf16", out_dtype="bf16", scale=1 / np.sqrt(128)), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    make, opts = CASES[name]
    case = make()
    dc = D.to_device(case, DEV)
    ws = torch.zeros(max(D.workspace_size(dc, opts), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty(tuple(case.q.shape), dtype=D.out_dtype(case), device=DEV)
    announce("graph %s: eager" % name)
    eager = D.run(dc, options=opts, out=out, workspace=ws).clone()     # also warms the launchers up
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    tol = "e4m3" if case.dtype == "e4m3" else "bf16"
    compare(eager, ref, tol, "graph %s eager" % name)
    announce("graph %s: capture" % name)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            D.run(dc, options=opts, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(4):
        announce("graph %s: replay %d" % (name, k))
        out.fill_(float("nan"))                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager call" % k
    del g
