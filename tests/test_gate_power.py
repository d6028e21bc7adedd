"""The GPU tests' parity gates reject plausible kernel mistakes (CPU only, no GPU).

Each case plants one mistake in the fp64 oracle's inputs and checks that the comparison
the GPU tests use (``gpu_util.compare``: max-abs and relative-RMS gates) rejects the
resulting output against the correct one. The mistakes: a key block of a block-sparse
row left out, 5 % of a row's listed keys left out, the latent attention sink ignored,
the K and V planes swapped, query head h read against kv head h mod Hkv instead of
h / group, the softmax scale applied twice. The correct output rounded to bf16 passes.
The attention outputs at these shapes are small (RMS 0.03-0.2), which is why the
max-abs bound alone would not catch most of these. Measured relative-RMS distances
against the 1e-2 gate: dropped block 0.49, 5 % of keys 0.24, sink ignored 0.019 (its
max-abs error 0.07 also exceeds 2e-2), scale applied twice 0.75; bf16 rounding of the
correct output 0.0017."""
import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import compare


def rejects(got: np.ndarray, ref: np.ndarray, dtype: str) -> bool:
    try:
        compare(torch.from_numpy(got), ref, dtype, "planted")
    except AssertionError:
        return True
    return False


def as_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).double().numpy()


def block_case():
    return W.make_block_sparse(name="gate_bs", seed=201, cache_lengths=[900, 2000, 300, 1500], rows=[1, 2, 1, 1],
                               page_size=128, num_kv_heads=2, group=8, head_dim=128, dtype="e4m3", topk=5,
                               block_size=64, scale=1 / np.sqrt(128), std=0.5)


def decode_case():
    return W.make_qsa(name="gate_qsa", seed=202, rows=[1] * 6, cache_lengths=[600, 900, 1200, 700, 2000, 1500],
                      page_size=128, num_layers=1, layer_idx=0, num_kv_heads=4, group=4, head_dim=128,
                      dtype="bf16", out_dtype="bf16", selection_width=512, selection="min", scale=1 / np.sqrt(128))


def latent_case():
    return W.make_latent(name="gate_latent", seed=203, decode_positions=[300, 1000, 77], prefill_positions=[500],
                         prefill_rows=9, num_heads=64, head_dim=512, dtype="bf16", out_dtype="bf16", window=24,
                         swa_page_size=16, comp_page_size=32, num_comp=40, comp_ratio=4, unused_frac=0.1,
                         scale=1 / np.sqrt(512))


@pytest.mark.parametrize("make,dtype", [(block_case, "e4m3"), (decode_case, "bf16"), (latent_case, "bf16")])
def test_correct_bf16_output_passes(make, dtype):
    case = make()
    ref = oracle.run_case(case)
    assert not rejects(as_bf16(ref), ref, dtype)


def test_dropped_key_block_is_rejected():
    case = block_case()
    ref = oracle.run_case(case)
    bad = copy.copy(case)
    bad.d_indices = case.d_indices.copy()
    # one block of five moved past every row's position (the causal clip then keeps none
    # of its keys): a block left out in every (kv head, row)
    bad.d_indices[:, :, 1] = 1 << 20
    assert rejects(oracle.run_case(bad), ref, "e4m3")


def test_five_percent_of_keys_dropped_is_rejected():
    case = decode_case()
    ref = oracle.run_case(case)
    bad = copy.copy(case)
    bad.counts = (case.counts * 95 // 100).astype(np.int32)
    assert rejects(oracle.run_case(bad), ref, "bf16")


def test_ignored_sink_is_rejected():
    case = latent_case()
    ref = oracle.run_case(case)
    bad = copy.copy(case)
    bad.attn_sink = np.full_like(np.asarray(case.attn_sink, np.float32), -1e30)
    assert rejects(oracle.run_case(bad), ref, "bf16")


def test_swapped_k_and_v_are_rejected():
    case = decode_case()
    ref = oracle.run_case(case)
    bad = copy.copy(case)
    kv = copy.copy(case.kv)
    kv.storage = case.kv.storage.clone()
    pv = kv.pages_view()
    k_plane = pv[:, 0].clone()
    pv[:, 0] = pv[:, 1]
    pv[:, 1] = k_plane
    bad.kv = kv
    assert rejects(oracle.run_case(bad), ref, "bf16")


def test_wrong_head_to_kv_head_mapping_is_rejected():
    case = decode_case()
    ref = oracle.run_case(case)
    hkv, G = case.kv.num_kv_heads, case.num_q_heads // case.kv.num_kv_heads
    # the output row of q head h computed as if h read kv head h mod Hkv: permute the
    # q heads, evaluate, and put the heads back in place
    perm = np.arange(hkv * G).reshape(G, hkv).T.reshape(-1)      # h -> position g*G + i with g = h mod Hkv
    bad = copy.copy(case)
    bad.q = case.q[:, perm].contiguous()
    got = oracle.run_case(bad)
    inv = np.argsort(perm)
    assert rejects(got[:, inv], ref, "bf16")


def test_scale_applied_twice_is_rejected():
    case = decode_case()
    ref = oracle.run_case(case)
    bad = copy.copy(case)
    bad.scale = float(np.float32(case.scale * case.scale))
    assert rejects(oracle.run_case(bad), ref, "bf16")
