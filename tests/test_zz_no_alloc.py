"""qsa_sparse_attention_no_alloc (split-K partials in the library's own device scratch
instead of a caller workspace) against qsa_sparse_attention with a workspace, through
the C ABI: same plan, same kernels, so the outputs must be bitwise equal, and both
within tolerance of the fp64 oracle. Each test makes two calls in a row on the shared
scratch, the second with a smaller input, so a stale partial of the first call would
show in the second."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_ragged_amd as qsa
import workloads as W
from workloads import device as D
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def decode(seed, batch, W_, hkv=8, g=4, d=128, dtype="bf16", out="bf16"):
    rng = np.random.default_rng(seed + 5000)
    cl = rng.integers(200, 3000, size=batch, endpoint=True)
    return W.make_qsa(name="decode_no_alloc", seed=seed, rows=[1] * batch, cache_lengths=cl, page_size=128,
                      num_layers=2, layer_idx=1, num_kv_heads=hkv, group=g, head_dim=d, dtype=dtype,
                      out_dtype=out, selection_width=W_, selection="uniform_counts", scale=1 / np.sqrt(d))


def prefill(seed, rows, cache, W_=256):
    return W.make_qsa(name="prefill_no_alloc", seed=seed, rows=list(rows), cache_lengths=list(cache),
                      page_size=128, num_layers=1, layer_idx=0, num_kv_heads=2, group=16, head_dim=128,
                      dtype="bf16", out_dtype="bf16", selection_width=W_, selection="recent", recent=64,
                      scale=1 / np.sqrt(128))


def check_pair(case, options, tol, what):
    dc = D.to_device(case, DEV)
    ws_n = D.workspace_size(dc, options)
    announce("%s: %d rows, workspace entry point needs %d bytes" % (what, case.total_q, ws_n))
    assert 0 < ws_n <= qsa.NO_ALLOC_SCRATCH_BYTES, "the case must use split-K partials that fit the scratch"
    ref_out = D.run(dc, options=options)
    c = dc.case
    got = torch.full_like(ref_out, float("nan"))
    qsa.sparse_attention_no_alloc(dc.q, dc.row_off, dc.kv, c.layer_idx, dc.token_indices, dc.counts, c.scale,
                                  out=got, max_prompt_length=c.max_prompt_length, options=options)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_out), "%s: no-alloc output differs from the workspace entry point" % what
    compare(got, oracle.run_case(case), tol, what)


# (case, options) of the first call, then of the second (smaller) call
PAIRS = {
    "bf16-decode-split": lambda: ((decode(101, 24, 1024), {"num_splits": 4}),
                                  (decode(102, 5, 300), {"num_splits": 3})),
    "bf16-decode-auto": lambda: ((decode(103, 16, 2048), None),              # automatic split plans
                                 (decode(104, 3, 700, hkv=2), None)),
    "bf16-prefill-mfma": lambda: ((prefill(105, (40, 70), (300, 900)), {"num_splits": 4}),
                                  (prefill(106, (9,), (60,)), {"num_splits": 2})),
    "f32-decode": lambda: ((decode(107, 6, 500, hkv=1, d=64, dtype="f32", out="f32"), {"num_splits": 7}),
                           (decode(108, 2, 90, hkv=1, d=64, dtype="f32", out="f32"), {"num_splits": 5})),
}


@pytest.mark.parametrize("name", list(PAIRS))
def test_no_alloc_matches_workspace_entry_point(name):
    for k, (case, options) in enumerate(PAIRS[name]()):
        tol = "f32" if case.dtype == "f32" else "bf16"
        check_pair(case, options, tol, "%s call %d" % (name, k + 1))


def test_no_alloc_refuses_plans_beyond_the_scratch():
    """A plan whose partials exceed the scratch is refused on the host with
    QSA_ERR_WORKSPACE, and the output is left untouched."""
    case = decode(109, 64, 2048)
    dc = D.to_device(case, DEV)
    opts = {"num_splits": 64}           # 64 splits x 64 rows x 32 heads x 130 fp32 = 68 MB
    assert D.workspace_size(dc, opts) > qsa.NO_ALLOC_SCRATCH_BYTES
    out = torch.full(tuple(case.q.shape), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_attention_no_alloc(dc.q, dc.row_off, dc.kv, case.layer_idx, dc.token_indices, dc.counts,
                                      case.scale, out=out, options=opts)
    assert e.value.status == 5 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
