"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle library handle (``oracle.load()`` or a deliberately
broken build) and raises AssertionError when the oracle disagrees with the pin.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
plants mistakes in copies of the oracle source and checks that some pin catches
every one of them.

Kinds of pin (none re-types the oracle's formula):
  * exhaustive codec checks against torch's CPU conversions and the format tables;
  * hand-derived closed-form cases (tests/golden/hand_cases.json);
  * brute force: numpy dense masked attention over a de-paged cache;
  * special cases that reduce to a library routine (torch's scaled_dot_product_attention
    with a causal or sliding-window mask, in float64 on the CPU);
  * invariants (page permutation, garbage past counts, index order, GQA expansion,
    sink as a closed-form factor, block-sparse as a token selection);
  * dense ragged attention (no cache) against torch SDPA with causal, sliding-window
    and empty masks per sequence, and the one-key closed forms.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


# ------------------------------------------------------------------ helpers

def dense_keys(cache: W.PagedCache, b: int, layer: int, T: int) -> np.ndarray:
    """[planes, T, Hkv, D] float64 of positions 0..T-1 of sequence b, read through the
    page table with torch indexing and decoded by torch's own dtype conversion."""
    if T == 0:
        return np.zeros((cache.planes, 0, cache.num_kv_heads, cache.head_dim))
    pv = cache.pages_view()
    npg = (T + cache.page_size - 1) // cache.page_size
    pages = torch.as_tensor(cache.lookup_table[b, :npg].astype(np.int64))
    x = pv[pages][:, :, layer]                                   # [npg, planes, ps, Hkv, D]
    x = x.permute(1, 0, 2, 3, 4).reshape(cache.planes, npg * cache.page_size,
                                         cache.num_kv_heads, cache.head_dim)[:, :T]
    return x.to(torch.float32).to(torch.float64).numpy()


def q64(case) -> np.ndarray:
    return case.q.to(torch.float32).to(torch.float64).numpy()


def masked_softmax_attend(qh, K, V, weight, scale, sink=-math.inf):
    """Dense masked attention: keys with weight 0 are masked out; weight w>0 counts a
    key w times. qh [H, D], K/V [T, D] (shared by the H heads)."""
    S = float(np.float32(scale)) * (qh @ K.T)                    # [H, T]
    live = weight > 0
    out = np.zeros((qh.shape[0], V.shape[1]))
    if not live.any():
        return out
    Sl = S[:, live]
    m = np.maximum(Sl.max(axis=1, keepdims=True), sink)
    E = weight[live][None, :] * np.exp(Sl - m)
    Z = E.sum(axis=1, keepdims=True) + np.exp(sink - m)
    return (E @ V[live]) / Z


def brute_qsa(case) -> np.ndarray:
    """numpy dense masked attention for the index-selected op (multiplicity-weighted mask)."""
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    off = case.input_row_offsets.astype(np.int64)
    Wd = case.token_indices.shape[1]
    qq = q64(case)
    out = np.zeros(qq.shape)
    for b in range(case.batch):
        T = int(kv.cache_lengths[b]) + int(off[b + 1] - off[b])
        KV = dense_keys(kv, b, case.layer_idx, T)
        for r in range(off[b], off[b + 1]):
            n = max(0, min(int(case.counts[r]), Wd))
            w = np.bincount(case.token_indices[r, :n].astype(np.int64), minlength=T)[:T].astype(np.float64)
            for g in range(kv.num_kv_heads):
                hs = slice(g * G, (g + 1) * G)
                out[r, hs] = masked_softmax_attend(qq[r, hs], KV[0, :, g], KV[1, :, g], w, case.scale)
    return out


def brute_block_sparse(case) -> np.ndarray:
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    off = case.input_row_offsets.astype(np.int64)
    pos = case.positions()
    bs = case.block_size
    qq = q64(case)
    out = np.zeros(qq.shape)
    for b in range(case.batch):
        T = int(pos[off[b + 1] - 1]) + 1
        KV = dense_keys(kv, b, case.layer_idx, T)
        for r in range(off[b], off[b + 1]):
            for g in range(kv.num_kv_heads):
                w = np.zeros(T)
                for blk in case.d_indices[g, r]:
                    lo = int(blk) * bs
                    hi = min(lo + bs, int(pos[r]) + 1)
                    if hi > lo:
                        w[lo:hi] += 1
                hs = slice(g * G, (g + 1) * G)
                out[r, hs] = masked_softmax_attend(qq[r, hs], KV[0, :, g], KV[1, :, g], w, case.scale)
    return out


def brute_latent(case, sink=None) -> np.ndarray:
    off = case.input_row_offsets.astype(np.int64)
    pos = case.positions()
    qq = q64(case)
    sink = case.attn_sink.astype(np.float64) if sink is None else sink
    out = np.zeros(qq.shape)
    for b in range(case.batch):
        T = int(pos[off[b + 1] - 1]) + 1
        X = dense_keys(case.kv, b, case.layer_idx, T)[0, :, 0]           # [T, D]
        E = int(case.comp_indices[off[b]:off[b + 1]].max(initial=-1)) + 1
        C = dense_keys(case.comp, b, case.layer_idx, E)[0, :, 0]          # [E, D]
        XC = np.concatenate([X, C], axis=0)
        for r in range(off[b], off[b + 1]):
            w = np.zeros(T + E)
            w[max(0, int(pos[r]) - case.window + 1): int(pos[r]) + 1] = 1
            ce = case.comp_indices[r]
            w[T:] += np.bincount(ce[ce >= 0].astype(np.int64), minlength=E)[:E]
            for h in range(case.num_q_heads):
                out[r, h] = masked_softmax_attend(qq[r, h][None], XC, XC, w, case.scale, sink[h])[0]
    return out


def assert_close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.isfinite(a).all(), what + ": oracle output has non-finite values"
    err = np.abs(a - b).max() if a.size else 0.0
    assert err <= tol, "%s: max abs diff %.3e > %.1e" % (what, err, tol)


def sdpa64(q, k, v, mask, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU (library routine)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q), torch.as_tensor(k), torch.as_tensor(v),
        attn_mask=torch.as_tensor(mask), scale=float(np.float32(scale))).numpy()


def clone_case(case, **kw):
    import copy
    c = copy.copy(case)
    c.kv = copy.copy(case.kv)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


# ------------------------------------------------------------------ small cases

def small_qsa_cases():
    """A spread of tiny shapes: dtypes, groups, kv heads, layers, padded pages, selections."""
    return [
        W.c1_tiny_fp32(),
        W.make_qsa(name="bf16_g2_h3_pad", seed=11, rows=[2, 1, 4], cache_lengths=[5, 0, 9],
                   page_size=4, num_layers=3, layer_idx=1, num_kv_heads=3, group=2, head_dim=8,
                   dtype="bf16", out_dtype="bf16", selection_width=7, selection="uniform_counts",
                   scale=0.3, spare_pages=2, page_pad=5),
        W.make_qsa(name="e4m3_g1_h2", seed=12, rows=[3, 2], cache_lengths=[12, 3], page_size=8,
                   num_layers=2, layer_idx=0, num_kv_heads=2, group=1, head_dim=16, dtype="e4m3",
                   out_dtype="bf16", selection_width=6, selection="min", scale=0.25, std=0.5),
        W.make_qsa(name="bf16_recent", seed=13, rows=[6], cache_lengths=[20], page_size=4,
                   num_layers=1, layer_idx=0, num_kv_heads=1, group=4, head_dim=8, dtype="bf16",
                   out_dtype="bf16", selection_width=12, selection="recent", recent=4, scale=0.4),
    ]


def small_block_sparse_case(seed=21, rows=None, cache_lengths=(40, 70, 13), topk=3, dtype="e4m3"):
    return W.make_block_sparse(name="bs_small", seed=seed, cache_lengths=list(cache_lengths), rows=rows,
                               page_size=8, num_kv_heads=2, group=3, head_dim=16, dtype=dtype,
                               topk=topk, block_size=4, scale=0.25, std=0.5, num_layers=2, layer_idx=1)


def small_latent_case(seed=31, unused=0.3):
    return W.make_latent(name="lat_small", seed=seed, decode_positions=[40, 13], prefill_positions=[25],
                         prefill_rows=5, num_heads=3, head_dim=16, dtype="bf16", out_dtype="bf16",
                         window=6, swa_page_size=4, comp_page_size=4, num_comp=5, comp_ratio=2,
                         unused_frac=unused, scale=0.25)


# ------------------------------------------------------------------ pins: codecs

def pin_bf16_codec_exhaustive(lib):
    codes = np.arange(65536, dtype=np.uint16)
    got = oracle.decode("bf16", codes, lib=lib)
    ref = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "bf16 NaN codes differ"
    assert (got[~nan] == ref[~nan]).all(), "bf16 decode differs from torch"
    # format definition, independent of torch: (-1)^s * 2^(e-127) * (1 + m/128), e in 1..254
    for c in (0x3F80, 0xC000, 0x0001, 0x7F7F, 0x4049, 0x8000, 0x0080):
        s, e, m = c >> 15, (c >> 7) & 0xFF, c & 0x7F
        v = (2.0 ** (e - 127)) * (1 + m / 128) if e else (2.0 ** -126) * (m / 128)
        v = -v if s else v
        assert got[c] == v, hex(c)
    assert got[0x7F80] == math.inf and got[0xFF80] == -math.inf


def pin_e4m3_codec_exhaustive(lib):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e4m3", codes, lib=lib)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (np.isnan(got) == nan).all(), "e4m3 NaN codes differ"
    assert (got[~nan] == ref[~nan]).all(), "e4m3 decode differs from torch"
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        assert got[c] == v, (hex(c), got[c], v)


def pin_f32_passthrough(lib):
    x = np.array([0.0, -1.5, 3.25e-40, 1e38, np.inf], np.float32)
    got = oracle.decode("f32", x, lib=lib)
    assert (got == x.astype(np.float64)).all()


# ------------------------------------------------------------------ pins: golden

def _golden_leaf(spec, D, planes, L, Hkv):
    n = spec["num_pages"]
    t = torch.full((n, planes, L, spec["page_size"], Hkv, D), float("nan"), dtype=torch.float32)
    for key, vals in spec["kv"].items():
        p, pl, l, s, h = (int(x) for x in key.split(","))
        t[p, pl, l, s, h] = torch.tensor(vals, dtype=torch.float32)
    return t


def pin_golden_hand_cases(lib):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        D, Hq = c["head_dim"], c["num_q_heads"]
        q = torch.tensor(c["q"], dtype=torch.float32)
        off = np.concatenate([[0], np.cumsum(c["rows"])]).astype(np.uint32)
        if c["op"] in ("qsa", "block_sparse"):
            Hkv, L = c["num_kv_heads"], c["num_layers"]
            blocks = _golden_leaf(c, D, 2, L, Hkv)
            common = dict(q=q, dtype="f32", input_row_offsets=off, kv_blocks=blocks,
                          num_pages=c["num_pages"], num_layers=L, page_size=c["page_size"],
                          num_kv_heads=Hkv, page_stride=-1, cache_lengths=c["cache_lengths"],
                          kv_lookup_table=np.array(c["lookup_table"]), layer_idx=c["layer_idx"],
                          scale=c["scale"], lib=lib)
            if c["op"] == "qsa":
                got = oracle.sparse_attention(token_indices=np.array(c["token_indices"]),
                                              counts=np.array(c["counts"]), **common)
            else:
                got = oracle.block_sparse_attention(d_indices=np.array(c["d_indices"]),
                                                    block_size=c["block_size"], **common)
        else:
            leaves = {}
            for name in ("swa", "comp"):
                sp = c[name]
                leaves[name] = dict(blocks=_golden_leaf(sp, D, 1, 1, 1), num_pages=sp["num_pages"],
                                    num_layers=1, page_size=sp["page_size"], page_stride=-1,
                                    kv_lookup_table=np.array(sp["lookup_table"]),
                                    cache_lengths=c["cache_lengths"])
            sink = np.array([float(x) for x in c["attn_sink"]], np.float32)
            got = oracle.latent_sparse_attention(q=q, dtype="f32", input_row_offsets=off,
                                                 swa=leaves["swa"], comp=leaves["comp"], layer_idx=0,
                                                 window=c["window"],
                                                 comp_indices=np.array(c["comp_indices"]),
                                                 attn_sink=sink, scale=c["scale"], lib=lib)
        assert_close(got, np.array(c["expected"]), 1e-15, "golden " + c["name"])


# ------------------------------------------------------------------ pins: qsa

def pin_qsa_brute_force(lib):
    for case in small_qsa_cases():
        got = oracle.run_case(case, lib=lib)
        assert_close(got, brute_qsa(case), 1e-12, "qsa brute force " + case.name)


def pin_qsa_duplicates_and_count_edges(lib):
    case = W.c1_tiny_fp32()
    idx = case.token_indices.copy()
    cnt = case.counts.copy()
    idx[1, :4] = [5, 5, 5, 9]                 # duplicates count with multiplicity
    cnt[1] = 4
    cnt[2] = 0                                # empty selection -> zero row
    cnt[3] = -3
    idx[4, :] = np.arange(16) % 30            # counts > width clamps to width
    cnt[4] = 99
    c2 = clone_case(case, token_indices=idx, counts=cnt)
    got = oracle.run_case(c2, lib=lib)
    assert (got[2] == 0).all() and (got[3] == 0).all()
    ref = brute_qsa(c2)
    assert_close(got, ref, 1e-12, "qsa duplicates/edges")


def pin_qsa_counts_one_exact(lib):
    case = small_qsa_cases()[1]
    cnt = np.ones_like(case.counts)
    c2 = clone_case(case, counts=cnt)
    got = oracle.run_case(c2, lib=lib)
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    off = case.input_row_offsets
    for b in range(case.batch):
        T = int(kv.cache_lengths[b]) + int(off[b + 1] - off[b])
        KV = dense_keys(kv, b, case.layer_idx, T)
        for r in range(off[b], off[b + 1]):
            p = case.token_indices[r, 0]
            for h in range(case.num_q_heads):
                assert (got[r, h] == KV[1, p, h // G]).all(), "counts=1 must return the V row exactly"


def pin_qsa_scale_zero_mean(lib):
    case = small_qsa_cases()[2]
    c2 = clone_case(case, scale=0.0)
    got = oracle.run_case(c2, lib=lib)
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    off = case.input_row_offsets
    for b in range(case.batch):
        T = int(kv.cache_lengths[b]) + int(off[b + 1] - off[b])
        KV = dense_keys(kv, b, case.layer_idx, T)
        for r in range(off[b], off[b + 1]):
            sel = case.token_indices[r, :case.counts[r]]
            for h in range(case.num_q_heads):
                assert_close(got[r, h], KV[1, sel, h // G].mean(axis=0), 1e-14, "scale=0 mean")


def pin_qsa_page_permutation(lib):
    case = small_qsa_cases()[1]
    base = oracle.run_case(case, lib=lib)
    rng = np.random.default_rng(99)
    kv = case.kv
    perm = rng.permutation(kv.num_pages)                 # old page i moves to perm[i]
    st = kv.storage.view(kv.num_pages, kv.page_elems)
    new = torch.empty_like(st)
    new[torch.as_tensor(perm)] = st
    import copy
    kv2 = copy.copy(kv)
    kv2.storage = new.view(-1)
    kv2.lookup_table = perm[kv.lookup_table.astype(np.int64)].astype(np.uint32)
    got = oracle.run_case(clone_case(case, kv=kv2), lib=lib)
    assert np.array_equal(got, base), "page permutation changed the oracle output"


def pin_qsa_garbage_past_counts(lib):
    case = small_qsa_cases()[0]
    base = oracle.run_case(case, lib=lib)
    assert np.isfinite(base).all()
    # poison: slots past counts name real, unselected positions whose K/V are set to NaN
    import copy
    kv = copy.copy(case.kv)
    kv.storage = case.kv.storage.clone()
    pv = kv.pages_view()
    idx = case.token_indices.copy()
    off = case.input_row_offsets
    for b in range(case.batch):
        T = int(kv.cache_lengths[b]) + int(off[b + 1] - off[b])
        used = set()
        for r in range(off[b], off[b + 1]):
            used |= set(case.token_indices[r, :case.counts[r]].tolist())
        free = [p for p in range(T) if p not in used]
        for p in free:
            pv[int(kv.lookup_table[b, p // kv.page_size]), :, case.layer_idx, p % kv.page_size] = float("nan")
        for r in range(off[b], off[b + 1]):
            n = case.counts[r]
            if free:
                idx[r, n:] = [free[k % len(free)] for k in range(idx.shape[1] - n)]
    got = oracle.run_case(clone_case(case, kv=kv, token_indices=idx), lib=lib)
    assert np.array_equal(got, base), "entries past counts influenced the output"


def pin_qsa_index_order(lib):
    case = small_qsa_cases()[1]
    base = oracle.run_case(case, lib=lib)
    rng = np.random.default_rng(5)
    idx = case.token_indices.copy()
    for r in range(case.total_q):
        n = case.counts[r]
        idx[r, :n] = rng.permutation(idx[r, :n])
    got = oracle.run_case(clone_case(case, token_indices=idx), lib=lib)
    assert_close(got, base, 1e-12, "index order")


def pin_qsa_gqa_expansion(lib):
    """Repeating each kv head `group` times and running with group 1 gives the same result."""
    case = small_qsa_cases()[1]
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    base = oracle.run_case(case, lib=lib)
    pv = kv.pages_view()
    rep = pv.repeat_interleave(G, dim=4).contiguous()
    import copy
    kv2 = copy.copy(kv)
    kv2.storage = rep.view(-1)
    kv2.num_kv_heads = kv.num_kv_heads * G
    kv2.page_stride = -1
    got = oracle.run_case(clone_case(case, kv=kv2), lib=lib)
    assert np.array_equal(got, base), "GQA expansion changed the output"


def pin_qsa_full_selection_is_causal_attention(lib):
    """Selecting every position 0..pos equals dense causal attention (torch SDPA, fp64)."""
    case = W.make_qsa(name="full", seed=14, rows=[4, 3], cache_lengths=[6, 2], page_size=4,
                      num_layers=1, layer_idx=0, num_kv_heads=2, group=2, head_dim=8, dtype="bf16",
                      out_dtype="bf16", selection_width=16, selection="min", scale=0.35)
    got = oracle.run_case(case, lib=lib)
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    off = case.input_row_offsets
    qq = q64(case)
    for b in range(case.batch):
        nr = int(off[b + 1] - off[b])
        T = int(kv.cache_lengths[b]) + nr
        KV = dense_keys(kv, b, 0, T)
        k = np.repeat(KV[0].transpose(1, 0, 2), G, axis=0)            # [Hq, T, D]
        v = np.repeat(KV[1].transpose(1, 0, 2), G, axis=0)
        qb = qq[off[b]:off[b + 1]].transpose(1, 0, 2)                  # [Hq, nr, D]
        posr = int(kv.cache_lengths[b]) + np.arange(nr)
        mask = np.arange(T)[None, :] <= posr[:, None]
        ref = sdpa64(qb, k, v, mask, case.scale).transpose(1, 0, 2)
        assert_close(got[off[b]:off[b + 1]], ref, 1e-12, "full selection vs SDPA")


# ------------------------------------------------------------------ pins: block-sparse

def pin_block_sparse_brute_force(lib):
    for case in (small_block_sparse_case(), small_block_sparse_case(seed=22, rows=[3, 1, 2], dtype="bf16")):
        got = oracle.run_case(case, lib=lib)
        assert_close(got, brute_block_sparse(case), 1e-12, "block-sparse brute force")


def pin_block_sparse_is_token_selection(lib):
    """Expanding block ids into per-kv-head token lists and running the index-selected op on
    one-kv-head slices gives bit-identical results."""
    case = small_block_sparse_case()
    got = oracle.run_case(case, lib=lib)
    kv = case.kv
    G = case.num_q_heads // kv.num_kv_heads
    pos = case.positions()
    bs = case.block_size
    pv = kv.pages_view()
    for g in range(kv.num_kv_heads):
        lists = []
        for r in range(case.total_q):
            toks = [int(blk) * bs + i for blk in case.d_indices[g, r] for i in range(bs)
                    if int(blk) * bs + i <= pos[r]]
            lists.append(toks)
        Wd = max(len(t) for t in lists)
        idx = np.full((case.total_q, Wd), -7, np.int32)
        for r, t in enumerate(lists):
            idx[r, :len(t)] = t
        sl = pv[:, :, :, :, g:g + 1].contiguous()
        out = oracle.sparse_attention(q=case.q[:, g * G:(g + 1) * G].contiguous(), dtype=case.dtype,
                                      input_row_offsets=case.input_row_offsets, kv_blocks=sl,
                                      num_pages=kv.num_pages, num_layers=kv.num_layers,
                                      page_size=kv.page_size, num_kv_heads=1, page_stride=-1,
                                      cache_lengths=kv.cache_lengths, kv_lookup_table=kv.lookup_table,
                                      layer_idx=case.layer_idx, token_indices=idx,
                                      counts=np.array([len(t) for t in lists], np.int32),
                                      scale=case.scale, lib=lib)
        assert np.array_equal(out, got[:, g * G:(g + 1) * G]), "block-sparse != token selection"


def pin_block_sparse_all_blocks_is_causal(lib):
    """Listing every block up to the row's position equals dense causal attention (SDPA).

    Row 0 (position 9) also lists block 3 (positions 12..15), which lies wholly after
    the row and must contribute nothing."""
    case = W.make_block_sparse(name="bs_all", seed=23, cache_lengths=[9, 15], page_size=8,
                               num_kv_heads=1, group=2, head_dim=8, dtype="bf16", topk=3,
                               block_size=4, scale=0.3, std=1.0)
    di = np.array([[[2, 0, 3, 1], [3, 1, 0, 2]]], np.int32)
    got = oracle.run_case(clone_case(case, d_indices=di), lib=lib)
    qq = q64(case)
    for r, T in ((0, 10), (1, 16)):
        KV = dense_keys(case.kv, r, 0, T)
        k = np.repeat(KV[0].transpose(1, 0, 2), 2, axis=0)
        v = np.repeat(KV[1].transpose(1, 0, 2), 2, axis=0)
        ref = sdpa64(qq[r:r + 1].transpose(1, 0, 2), k, v, np.ones((1, T), bool),
                     case.scale).transpose(1, 0, 2)
        assert_close(got[r:r + 1], ref, 1e-12, "all blocks vs SDPA row %d" % r)


# ------------------------------------------------------------------ pins: latent

def pin_latent_brute_force(lib):
    for case in (small_latent_case(), small_latent_case(seed=32, unused=0.0)):
        got = oracle.run_case(case, lib=lib)
        assert_close(got, brute_latent(case), 1e-12, "latent brute force")


def pin_latent_window_only_is_sliding_window_attention(lib):
    """No compressed entries and no sink equals sliding-window causal attention (SDPA)."""
    case = small_latent_case(seed=33)
    ci = np.full_like(case.comp_indices, -1)
    sink = np.full(case.num_q_heads, -np.inf, np.float32)
    got = oracle.run_case(clone_case(case, comp_indices=ci, attn_sink=sink), lib=lib)
    off = case.input_row_offsets
    pos = case.positions()
    qq = q64(case)
    for b in range(case.batch):
        T = int(pos[off[b + 1] - 1]) + 1
        X = dense_keys(case.kv, b, 0, T)[0, :, 0]
        pr = pos[off[b]:off[b + 1]]
        p = np.arange(T)[None, :]
        mask = (p <= pr[:, None]) & (p > pr[:, None] - case.window)
        # positions outside every window hold NaN in the leaf; they are masked out, so
        # zero them for the library routine (0 weight times NaN would still be NaN)
        X = np.where(np.isnan(X), 0.0, X)
        x = np.ascontiguousarray(np.broadcast_to(X, (case.num_q_heads, T, X.shape[1])))
        ref = sdpa64(qq[off[b]:off[b + 1]].transpose(1, 0, 2), x, x, mask, case.scale).transpose(1, 0, 2)
        assert_close(got[off[b]:off[b + 1]], ref, 1e-12, "window-only vs SDPA")


def pin_latent_sink_factor(lib):
    """out_with_sink = out_without_sink * sigmoid(LSE(scores) - sink), per row and head."""
    case = small_latent_case(seed=34)
    nos = np.full(case.num_q_heads, -np.inf, np.float32)
    with_sink = oracle.run_case(case, lib=lib)
    without = oracle.run_case(clone_case(case, attn_sink=nos), lib=lib)
    off = case.input_row_offsets
    pos = case.positions()
    qq = q64(case)
    sc = float(np.float32(case.scale))
    for b in range(case.batch):
        T = int(pos[off[b + 1] - 1]) + 1
        X = dense_keys(case.kv, b, 0, T)[0, :, 0]
        E = int(case.comp_indices[off[b]:off[b + 1]].max(initial=-1)) + 1
        C = dense_keys(case.comp, b, 0, E)[0, :, 0]
        for r in range(off[b], off[b + 1]):
            keys = [X[p] for p in range(max(0, int(pos[r]) - case.window + 1), int(pos[r]) + 1)]
            keys += [C[e] for e in case.comp_indices[r] if e >= 0]
            Kr = np.stack(keys)
            for h in range(case.num_q_heads):
                s = sc * (Kr @ qq[r, h])
                lse = s.max() + math.log(np.exp(s - s.max()).sum())
                f = 1.0 / (1.0 + math.exp(float(case.attn_sink[h]) - lse))
                assert_close(with_sink[r, h], without[r, h] * f, 1e-13, "sink factor")


def pin_latent_unused_slots_anywhere(lib):
    """-1 slots are skipped wherever they sit: compacting them to the tail changes nothing."""
    case = small_latent_case(seed=35, unused=0.4)
    base = oracle.run_case(case, lib=lib)
    ci = np.full_like(case.comp_indices, -1)
    for r in range(case.total_q):
        v = case.comp_indices[r][case.comp_indices[r] >= 0]
        ci[r, :len(v)] = v
    got = oracle.run_case(clone_case(case, comp_indices=ci), lib=lib)
    assert np.array_equal(got, base)


# ------------------------------------------------------------------ pins: dense ragged

def _dense_sdpa(case, mask_of):
    """Per sequence: torch SDPA in float64 with GQA expanded by repetition and the mask
    mask_of(i, j) over the sequence's own rows (i) and keys (j)."""
    off = case.input_row_offsets
    G = case.num_q_heads // case.k.shape[1]
    q = q64(case)
    k = case.k.to(torch.float32).to(torch.float64).numpy()
    v = case.v.to(torch.float32).to(torch.float64).numpy()
    out = np.zeros_like(q)
    for b in range(case.batch):
        a0, a1 = int(off[b]), int(off[b + 1])
        L = a1 - a0
        if L == 0:
            continue
        i = np.arange(L)[:, None]
        j = np.arange(L)[None, :]
        kk = np.repeat(k[a0:a1].transpose(1, 0, 2), G, axis=0)
        vv = np.repeat(v[a0:a1].transpose(1, 0, 2), G, axis=0)
        ref = sdpa64(q[a0:a1].transpose(1, 0, 2), kk, vv, mask_of(i, j), case.scale)
        out[a0:a1] = ref.transpose(1, 0, 2)
    return out


def _dense_case(seed, rows, causal, window, hkv=2, group=2, d=16, dtype="bf16"):
    return W.make_dense(name="dense_pin", seed=seed, rows=rows, num_kv_heads=hkv, group=group, head_dim=d,
                        dtype=dtype, out_dtype="f32", causal=causal, window=window, scale=0.3)


def pin_dense_causal_is_sdpa(lib):
    """Causal dense ragged attention equals torch SDPA with a lower-triangular mask per
    sequence (keys of other sequences never enter)."""
    case = _dense_case(41, [7, 1, 12, 4], True, -1)
    got = oracle.run_case(case, lib=lib)
    assert_close(got, _dense_sdpa(case, lambda i, j: j <= i), 1e-12, "dense causal vs SDPA")


def pin_dense_no_mask_is_sdpa(lib):
    case = _dense_case(42, [5, 9, 3], False, -1, hkv=1, group=4, dtype="f32")
    got = oracle.run_case(case, lib=lib)
    assert_close(got, _dense_sdpa(case, lambda i, j: np.ones_like(i + j, bool)), 1e-12, "dense no mask vs SDPA")


def pin_dense_sliding_window_is_sdpa(lib):
    """A local window w keeps keys i - w + 1 <= j (with j <= i under the causal mask)."""
    for w in (1, 3, 6):
        case = _dense_case(43 + w, [11, 2, 8], True, w, hkv=2, group=1)
        got = oracle.run_case(case, lib=lib)
        ref = _dense_sdpa(case, lambda i, j, w=w: (j <= i) & (j >= i - w + 1))
        assert_close(got, ref, 1e-12, "dense window %d vs SDPA" % w)
    case = _dense_case(49, [9, 5], False, 3, hkv=1, group=2)
    got = oracle.run_case(case, lib=lib)
    assert_close(got, _dense_sdpa(case, lambda i, j: j >= i - 2), 1e-12, "dense window, no causal mask")


def pin_dense_first_row_and_unit_window_are_v_rows(lib):
    """Closed forms: the first row of a causal sequence and every row under a window of
    one see exactly one key, so their output is that key's V row (every q head)."""
    case = _dense_case(50, [6, 3], True, 1, hkv=2, group=3, d=8, dtype="f32")
    got = oracle.run_case(case, lib=lib)
    v = case.v.double().numpy()
    G = 3
    for r in range(case.total_q):
        for h in range(case.num_q_heads):
            assert_close(got[r, h], v[r, h // G], 0.0, "window 1 row %d head %d" % (r, h))


# ------------------------------------------------------------------ pins: key compression

def small_compress_case(seed=41, dtype="bf16", freq_dtype="f32", ratio=4, rotary_dim=8, D=16, eps=1e-6,
                        cache_lengths=(13, 30, 0, 7), rows=(3, 1, 2, 1), **kw):
    return W.make_compress(name="compress_pin", seed=seed, cache_lengths=list(cache_lengths), rows=list(rows),
                           page_size=8, num_layers=2, layer_idx=1, head_dim=D, dtype=dtype,
                           freq_dtype=freq_dtype, ratio=ratio, rotary_dim=rotary_dim, eps=eps, **kw)


def torch_compress(case) -> np.ndarray:
    """The block keys from library routines, in float64: raw keys de-paged with torch
    indexing, each complete group averaged by Tensor.mean, torch's rms_norm with gamma,
    and the rotation as a product of complex numbers (view_as_complex). Rows past a
    sequence's block count are NaN, as in the oracle."""
    D, R, rd, mb = case.head_dim, case.ratio, case.rotary_dim, case.max_blocks
    out = np.full((case.batch * mb, D), np.nan)
    g = case.gamma.to(torch.float32).to(torch.float64)
    for b, nb in enumerate(case.blocks_per_sequence()):
        nb = int(nb)
        if nb == 0:
            continue
        K = torch.from_numpy(dense_keys(case.kv, b, case.layer_idx, nb * R)[0, :, 0, :])
        x = K.reshape(nb, R, D).mean(dim=1)
        y = torch.nn.functional.rms_norm(x, (D,), weight=g, eps=case.eps)
        if rd:
            f = case.freqs.to(torch.float32).to(torch.float64)[torch.arange(nb) * R]
            z = torch.view_as_complex(y[:, :rd].reshape(nb, rd // 2, 2).contiguous()) * \
                torch.view_as_complex(f.reshape(nb, rd // 2, 2).contiguous())
            y = torch.cat([torch.view_as_real(z).reshape(nb, rd), y[:, rd:]], dim=1)
        out[b * mb:b * mb + nb] = y.numpy()
    return out


def assert_same_rows(got, ref, tol, what):
    """Equal NaN pattern (rows not produced) and close values elsewhere."""
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), what + ": rows produced differ"
    live = ~np.isnan(ref)
    err = np.abs(got[live] - ref[live]).max() if live.any() else 0.0
    assert err <= tol, "%s: max abs diff %.3e > %.1e" % (what, err, tol)


def pin_compress_matches_library_pipeline(lib):
    cases = [
        small_compress_case(),
        small_compress_case(seed=42, dtype="f32", freq_dtype="bf16", ratio=3, rotary_dim=16),
        small_compress_case(seed=43, ratio=1, rotary_dim=0, eps=0.5),
        small_compress_case(seed=44, dtype="f32", ratio=5, rotary_dim=6, D=32, page_pad=3,
                            cache_lengths=(40, 9, 22), rows=(1, 1, 4)),
        small_compress_case(seed=45, ratio=8, rotary_dim=16, max_blocks=3),     # capped block count
    ]
    for case in cases:
        assert_same_rows(oracle.run_case(case, lib=lib), torch_compress(case), 1e-12,
                         "compress %s ratio=%d rd=%d" % (case.dtype, case.ratio, case.rotary_dim))


def pin_compress_closed_form(lib):
    """Hand-derived case, D 4, ratio 2, rotary 2, eps 0.5, gamma (2, 1, 0.5, 1): the two
    raw keys of each block are u + e and u - e with u = (3, 0, 1, -1), so the mean is u,
    mean(u^2) + eps = 11/4 + 1/2 = 13/4, and the normed key is gamma * u * 2/sqrt(13) =
    (6, 0, 0.5, -1) * 2/sqrt(13). The table row p holds (cos, sin) of 0.1 * (p + 1), and
    block j uses row 2j: the first pair (6k, 0) turns into (6k cos, 6k sin) of that angle;
    channels 2 and 3 are not rotated."""
    case = small_compress_case(seed=46, dtype="f32", ratio=2, rotary_dim=2, D=4, eps=0.5,
                               cache_lengths=(5,), rows=(1,))
    u = np.array([3.0, 0.0, 1.0, -1.0])
    e = np.array([1.0, 2.0, -0.5, 0.25])
    pv = case.kv.pages_view()
    for p in range(6):
        val = u + e if p % 2 == 0 else u - e
        pv[int(case.kv.lookup_table[0, p // case.kv.page_size]), 0, case.layer_idx, p % case.kv.page_size, 0] = \
            torch.as_tensor(val, dtype=torch.float32)
    case.gamma = torch.tensor([2.0, 1.0, 0.5, 1.0])
    ang = 0.1 * (np.arange(case.freqs.shape[0]) + 1)
    case.freqs = torch.as_tensor(np.stack([np.cos(ang), np.sin(ang)], 1), dtype=torch.float32)
    got = oracle.run_case(case, lib=lib)
    k = 2.0 / math.sqrt(13.0)
    f = case.freqs.to(torch.float64).numpy()
    for j in range(3):
        c, s = f[2 * j]
        assert_close(got[j], [6 * k * c, 6 * k * s, 0.5 * k, -k], 1e-12, "compress closed form block %d" % j)
    assert np.isnan(got[3:]).all(), "compress closed form: rows past the block count"


def pin_compress_page_permutation(lib):
    case = small_compress_case(seed=47, page_pad=2)
    base = oracle.run_case(case, lib=lib)
    kv = case.kv
    perm = np.random.default_rng(98).permutation(kv.num_pages)
    st = kv.storage.view(kv.num_pages, kv.page_elems)
    new = torch.empty_like(st)
    new[torch.as_tensor(perm)] = st
    import copy
    kv2 = copy.copy(kv)
    kv2.storage = new.view(-1)
    kv2.lookup_table = perm[kv.lookup_table.astype(np.int64)].astype(np.uint32)
    c2 = copy.copy(case)
    c2.kv = kv2
    got = oracle.run_case(c2, lib=lib)
    assert np.array_equal(np.isnan(got), np.isnan(base)) and np.array_equal(got[~np.isnan(got)],
                                                                              base[~np.isnan(base)]), \
        "page permutation changed the block keys"


def pin_compress_reads_complete_groups_only(lib):
    """NaN at every position of a trailing partial group (and past the key count): the
    produced block keys are unchanged and finite; zero and negative key counts give no
    block key."""
    case = small_compress_case(seed=48, ratio=4, cache_lengths=(13, 30, 5, 7), rows=(3, 1, 2, 1))
    base = oracle.run_case(case, lib=lib)
    import copy
    c2 = copy.copy(case)
    c2.kv = copy.copy(case.kv)
    c2.kv.storage = case.kv.storage.clone()
    pv = c2.kv.pages_view()
    for b, nb in enumerate(case.blocks_per_sequence()):
        for p in range(int(nb) * case.ratio, case.kv.max_pages * case.kv.page_size):
            pv[int(c2.kv.lookup_table[b, p // case.kv.page_size]), 0, case.layer_idx, p % case.kv.page_size] = \
                float("nan")
    got = oracle.run_case(c2, lib=lib)
    live = ~np.isnan(base)
    assert live.any() and np.array_equal(np.isnan(got), ~live) and np.array_equal(got[live], base[live]), \
        "compress read a raw key outside the complete groups"
    c3 = copy.copy(case)
    c3.key_counts = np.array([0, -5, 3, 4], np.int32)
    got = oracle.run_case(c3, lib=lib).reshape(4, case.max_blocks, -1)
    assert np.isnan(got[:3]).all() and np.isfinite(got[3, 0]).all() and np.isnan(got[3, 1:]).all(), \
        "compress block counts from zero, negative and short key counts"


def pin_compress_scale_invariance_without_eps(lib):
    """With eps 0 the RMS norm cancels any common scale of the raw keys: multiplying
    them all by 4 (exact in bf16) leaves the block keys unchanged."""
    case = small_compress_case(seed=49, eps=0.0)
    base = oracle.run_case(case, lib=lib)
    import copy
    c2 = copy.copy(case)
    c2.kv = copy.copy(case.kv)
    c2.kv.storage = case.kv.storage * 4
    assert_same_rows(oracle.run_case(c2, lib=lib), base, 1e-12, "compress scale invariance")


# ------------------------------------------------------------------ pins: block selection

def small_select_cases():
    return [
        W.make_select(name="sel_int", seed=51, rows=[1, 3, 2, 1], cache_lengths=[40, 23, 2, 77], head_dim=16,
                      dtype="bf16", ratio=4, topk=5, integer=True),
        W.make_select(name="sel_f32", seed=52, rows=[2, 1, 4], cache_lengths=[100, 9, 60], head_dim=32,
                      dtype="f32", ratio=3, topk=7),
        W.make_select(name="sel_cap", seed=53, rows=[1, 2], cache_lengths=[90, 200], head_dim=8, dtype="bf16",
                      ratio=4, topk=6, max_blocks=20, integer=True),
        W.make_select(name="sel_r1", seed=54, rows=[3, 1], cache_lengths=[12, 0], head_dim=16, dtype="bf16",
                      ratio=1, topk=4, W=9),
    ]


def numpy_select(case):
    """Selection from library routines: fp64 scores by numpy matrix products and the
    order (score descending, block index ascending) by numpy.lexsort."""
    q = case.q_index.to(torch.float32).to(torch.float64).numpy()
    bk = case.block_keys.to(torch.float32).to(torch.float64).numpy().reshape(case.batch, case.max_blocks, -1)
    off = case.input_row_offsets.astype(np.int64)
    pos = case.positions()
    rows = []
    for r in range(case.total_q):
        b = int(np.searchsorted(off, r, side="right") - 1)
        nfull = (pos[r] + 1) // case.ratio
        nv = min(nfull, case.max_blocks)
        s = bk[b, :nv] @ q[r]
        order = np.lexsort((np.arange(nv), -s))
        kept = np.sort(order[:min(case.topk, nv)])
        toks = [int(j) * case.ratio + t for j in kept for t in range(case.ratio)]
        toks += list(range(nfull * case.ratio, pos[r] + 1))
        rows.append((toks, kept))
    return rows


def check_select(case, got, what):
    idx, counts, blocks = got
    for r, (toks, kept) in enumerate(numpy_select(case)):
        assert counts[r] == len(toks), "%s row %d: count %d != %d" % (what, r, counts[r], len(toks))
        assert idx[r, :counts[r]].tolist() == toks, "%s row %d: token indices differ" % (what, r)
        assert (idx[r, counts[r]:] == -7).all(), "%s row %d: wrote past the count" % (what, r)
        exp = list(kept) + [-1] * (case.topk - len(kept))
        assert blocks[r].tolist() == exp, "%s row %d: blocks %s != %s" % (what, r, blocks[r].tolist(), exp)


def pin_select_matches_numpy_lexsort(lib):
    for case in small_select_cases():
        check_select(case, oracle.run_case(case, lib=lib), case.name)


def pin_select_closed_forms(lib):
    """A zero query scores every block 0: the first k blocks win (ties go to the lower
    index). A row before its first complete group keeps only its own positions. A
    planted block (the query itself, scaled up) always wins."""
    case = W.make_select(name="sel_zero", seed=55, rows=[1, 1, 1], cache_lengths=[50, 2, 30], head_dim=16,
                         dtype="f32", ratio=4, topk=3)
    case.q_index = torch.zeros_like(case.q_index)
    idx, counts, blocks = oracle.run_case(case, lib=lib)
    assert blocks[0].tolist() == [0, 1, 2] and counts[0] == 12 + 3           # pos 50: 12 complete, 3 tail
    assert idx[0, :15].tolist() == list(range(12)) + [48, 49, 50]
    assert counts[1] == 3 and idx[1, :3].tolist() == [0, 1, 2] and blocks[1].tolist() == [-1, -1, -1]
    case = W.make_select(name="sel_plant", seed=56, rows=[1], cache_lengths=[200], head_dim=16, dtype="f32",
                         ratio=4, topk=1)
    case.block_keys = case.block_keys.clone()
    case.block_keys[37] = case.q_index[0] * 8
    idx, counts, blocks = oracle.run_case(case, lib=lib)
    assert blocks[0].tolist() == [37] and idx[0, :4].tolist() == [148, 149, 150, 151]


def pin_select_positive_scale_invariance(lib):
    for case in small_select_cases()[:2]:
        base = oracle.run_case(case, lib=lib)
        c2 = W.SelectCase(**{**case.__dict__, "q_index": case.q_index * 4})
        got = oracle.run_case(c2, lib=lib)
        assert all(np.array_equal(a, b) for a, b in zip(base, got)), "scaling the query changed the selection"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
