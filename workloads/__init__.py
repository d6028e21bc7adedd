"""Seeded synthetic inputs for index-selected sparse attention over a paged KV cache.

This module only *draws inputs*; it computes nothing of the attention method.
Both the fp64 CPU oracle (``oracle/``) and the HIP path consume the exact same
bytes produced here, so parity compares like with like.

Tensor contracts follow the "Tensor shapes" lists of the pages
"QSASparseAttentionRaggedPaged" (q, input_row_offsets, kv_blocks, cache_lengths,
kv_lookup_table, token_indices, counts), "Struct_msa_attention_ragged_paged"
(d_indices [n_kv_heads, num_rows, topk]) and "latent_sparse_attention_ragged_paged"
(comp_indices, attn_sink, a token-paged window leaf and an entry-paged compressed
leaf, one latent head each).

Recipe conventions (stated once, used by every generator):

* Metadata (lengths, counts, indices, page permutation) come from
  ``numpy.random.default_rng(seed)``.
* Values come from torch CPU generators seeded from (seed, stream tag, chunk),
  drawn as N(0, std^2) float32 and cast by torch on the CPU to the storage dtype
  (round to nearest even; e4m3 is torch's ``float8_e4m3fn``).
* Row r of sequence b sits at position ``cache_lengths[b] + (r - input_row_offsets[b])``
  and the cache already holds positions ``0 .. that position`` (this step's keys
  included), which is how the key-compression page describes its key counts.
* Cache slots that no sequence may read (positions past a sequence's last
  position, spare pages, layers other than the addressed one, window-leaf
  positions no row's window reaches) are filled with NaN, so any stray read
  shows up in the output.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}

_CHUNK = 1 << 24


def _normal(shape, seed: int, tag: int, std: float, dtype: str) -> torch.Tensor:
    """N(0, std^2) values of ``shape`` cast to ``dtype``; deterministic in (seed, tag).

    Large draws are split into fixed 16M-element chunks, each with its own
    generator, so the result does not depend on the number of worker threads.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=TORCH_DTYPE[dtype])
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = torch.Generator().manual_seed((seed * 1000003 + tag * 7919 + c) & 0x7FFFFFFFFFFF)
        v = torch.randn(hi - lo, generator=g, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        out[lo:hi] = v.to(out.dtype)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(max_workers=min(8, nchunks)) as ex:
            list(ex.map(work, range(nchunks)))
    return out.view(*shape)


def nan_fill_(t: torch.Tensor) -> torch.Tensor:
    """Fill ``t`` in place with NaN (0x7F for e4m3, whose format has no infinity)."""
    if t.dtype == torch.float8_e4m3fn:
        t.view(torch.uint8).fill_(0x7F)
    else:
        t.fill_(float("nan"))
    return t


@dataclass
class PagedCache:
    """One paged cache leaf: blocks [num_pages, planes, num_layers, page_size, num_kv_heads, head_dim].

    ``storage`` is a flat tensor of ``num_pages * page_elems`` elements where
    ``page_elems`` is the packed page size, or ``page_stride`` when that is not -1
    (pages then carry ``page_stride - packed`` padding elements at their end).
    """
    storage: torch.Tensor
    dtype: str
    num_pages: int
    planes: int
    num_layers: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    page_stride: int            # -1 = packed
    lookup_table: np.ndarray    # [batch, max_pages] uint32
    cache_lengths: np.ndarray   # [batch] uint32
    max_cache_length: int

    @property
    def packed_page_elems(self) -> int:
        return self.planes * self.num_layers * self.page_size * self.num_kv_heads * self.head_dim

    @property
    def page_elems(self) -> int:
        return self.packed_page_elems if self.page_stride == -1 else self.page_stride

    @property
    def max_pages(self) -> int:
        return self.lookup_table.shape[1]

    def pages_view(self) -> torch.Tensor:
        """[num_pages, planes, L, ps, Hkv, D] view (padding excluded)."""
        v = self.storage.view(self.num_pages, self.page_elems)[:, : self.packed_page_elems]
        return v.view(self.num_pages, self.planes, self.num_layers, self.page_size,
                      self.num_kv_heads, self.head_dim)


@dataclass
class Case:
    """One call's worth of inputs. ``kind`` is "qsa", "block_sparse", "latent" or "dense"."""
    kind: str
    name: str
    seed: int
    dtype: str                       # q and kv element type
    out_dtype: str
    q: torch.Tensor                  # [total_q, Hq, D]
    input_row_offsets: np.ndarray    # [batch+1] uint32
    max_prompt_length: int
    kv: Optional[PagedCache]         # qsa/block_sparse: the K/V cache; latent: the window leaf; dense: None
    layer_idx: int
    scale: float
    # qsa
    token_indices: Optional[np.ndarray] = None   # [total_q, W] int32
    counts: Optional[np.ndarray] = None          # [total_q] int32
    # block-sparse
    d_indices: Optional[np.ndarray] = None       # [Hkv, total_q, topk] int32
    block_size: int = 0
    # latent
    comp: Optional[PagedCache] = None
    window: int = 0
    comp_indices: Optional[np.ndarray] = None    # [total_q, num_comp] int32
    attn_sink: Optional[np.ndarray] = None       # [Hq] float32
    # dense (no cache): k, v [total_q, Hkv, D]; causal mask; window (latent too) <= 0: none
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    causal: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return self.q.shape[0]

    @property
    def batch(self) -> int:
        return len(self.input_row_offsets) - 1

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    def positions(self) -> np.ndarray:
        """Position of every query row (input recipe convention, see module doc)."""
        off = self.input_row_offsets.astype(np.int64)
        pos = np.empty(self.total_q, np.int64)
        for b in range(self.batch):
            pos[off[b]:off[b + 1]] = int(self.kv.cache_lengths[b]) + np.arange(off[b + 1] - off[b])
        return pos


# --------------------------------------------------------------------------- pools

def _page_pool(rng, pages_needed: List[int], spare: int, max_pages: Optional[int] = None):
    """Shuffled physical page pool; returns (lut [batch, max_pages] uint32, num_pages, spare ids)."""
    total = int(sum(pages_needed)) + spare
    perm = rng.permutation(total).astype(np.int64)
    mp = max(1, max(pages_needed) if max_pages is None else max_pages)
    spare_ids = perm[sum(pages_needed):]
    fill = int(spare_ids[0]) if spare > 0 else 0
    lut = np.full((len(pages_needed), mp), fill, dtype=np.uint32)
    cur = 0
    for b, n in enumerate(pages_needed):
        lut[b, :n] = perm[cur:cur + n]
        cur += n
    return lut, total, spare_ids


def _fill_cache(cache: PagedCache, seed: int, tag: int, std: float, valid_ranges, layer: int):
    """Give positions [lo, hi] of each sequence random values in ``layer``; everything else NaN.

    ``valid_ranges[b] = (lo, hi)`` (inclusive). Values for sequence b are drawn as one
    [planes, hi-lo+1, Hkv, D] block from the (seed, tag*4096+b) stream.
    """
    nan_fill_(cache.storage)
    pv = cache.pages_view()
    ps = cache.page_size
    work = [(b, lo, hi) for b, (lo, hi) in enumerate(valid_ranges) if hi >= lo]

    def draw(item):
        b, lo, hi = item
        return b, lo, hi, _normal((cache.planes, hi - lo + 1, cache.num_kv_heads, cache.head_dim),
                                  seed, tag * 4096 + b, std, cache.dtype)

    with ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(draw, work))
    for b, lo, hi, vals in results:
        p = lo
        while p <= hi:
            lp = p // ps
            s0 = p % ps
            n = min(ps - s0, hi - p + 1)
            phys = int(cache.lookup_table[b, lp])
            pv[phys, :, layer, s0:s0 + n] = vals[:, p - lo:p - lo + n]
            p += n


def _make_cache(rng, dtype, planes, num_layers, ps, hkv, d, tokens, spare, page_pad=0,
                cache_lengths=None, max_pages=None, logical_pages=None):
    """Allocate a pool sized for ``tokens[b]`` positions per sequence (logical pages 0..)."""
    need = [max(1, math.ceil(t / ps)) for t in tokens] if logical_pages is None else logical_pages
    lut, num_pages, spare_ids = _page_pool(rng, need, spare, max_pages)
    packed = planes * num_layers * ps * hkv * d
    page_stride = -1 if page_pad == 0 else packed + page_pad
    per = packed if page_stride == -1 else page_stride
    storage = torch.empty(num_pages * per, dtype=TORCH_DTYPE[dtype])
    cl = np.zeros(len(tokens), np.uint32) if cache_lengths is None else np.asarray(cache_lengths, np.uint32)
    c = PagedCache(storage, dtype, num_pages, planes, num_layers, ps, hkv, d, page_stride,
                   lut, cl, int(cl.max()) if len(cl) else 0)
    return c, spare_ids


def _row_offsets(rows):
    off = np.zeros(len(rows) + 1, np.uint32)
    off[1:] = np.cumsum(rows)
    return off


# --------------------------------------------------------------------------- qsa

def make_qsa(*, name="qsa", seed, rows, cache_lengths, page_size, num_layers, layer_idx,
             num_kv_heads, group, head_dim, dtype, out_dtype, selection_width, selection,
             scale, spare_pages=4, page_pad=0, std=1.0, fill_past=-7, recent=64) -> Case:
    """Index-selected sparse GQA inputs ("QSASparseAttentionRaggedPaged" tensor shapes).

    selection:
      "uniform_counts": counts ~ U[1, min(W, pos+1)], distinct sorted indices in [0, pos];
      "min":            counts = min(W, pos+1), distinct sorted indices in [0, pos];
      "recent":         counts = min(W, pos+1): the last min(recent, pos+1) positions plus
                        distinct uniform earlier ones, sorted.
    Slots at or past counts hold ``fill_past``.
    """
    rng = np.random.default_rng(seed)
    rows = [int(x) for x in rows]
    cache_lengths = [int(x) for x in cache_lengths]
    batch = len(rows)
    tokens = [cache_lengths[b] + rows[b] for b in range(batch)]
    kv, _ = _make_cache(rng, dtype, 2, num_layers, page_size, num_kv_heads, head_dim, tokens,
                        spare_pages, page_pad, cache_lengths)
    off = _row_offsets(rows)
    total_q = int(off[-1])
    W = int(selection_width)
    idx = np.full((total_q, W), fill_past, np.int32)
    counts = np.zeros(total_q, np.int32)
    for b in range(batch):
        for i in range(rows[b]):
            r = int(off[b]) + i
            pos = cache_lengths[b] + i
            if selection == "uniform_counts":
                n = int(rng.integers(1, min(W, pos + 1), endpoint=True))
                sel = np.sort(rng.choice(pos + 1, n, replace=False))
            elif selection == "min":
                n = min(W, pos + 1)
                sel = np.sort(rng.choice(pos + 1, n, replace=False))
            elif selection == "recent":
                n = min(W, pos + 1)
                nr = min(recent, n)
                tail = np.arange(pos + 1 - nr, pos + 1)
                early = rng.choice(pos + 1 - nr, n - nr, replace=False) if n > nr else np.zeros(0, np.int64)
                sel = np.sort(np.concatenate([early, tail]))
            else:
                raise ValueError(selection)
            counts[r] = n
            idx[r, :n] = sel
    _fill_cache(kv, seed, 1, std, [(0, t - 1) for t in tokens], layer_idx)
    q = _normal((total_q, num_kv_heads * group, head_dim), seed, 2, std, dtype)
    return Case("qsa", name, seed, dtype, out_dtype, q, off, max(rows), kv, layer_idx,
                float(np.float32(scale)), token_indices=idx, counts=counts,
                meta={"group": group, "selection": selection})


# --------------------------------------------------------------------------- block-sparse

def make_block_sparse(*, name="block_sparse", seed, cache_lengths, page_size, num_kv_heads,
                      group, head_dim, dtype, topk, block_size, scale, rows=None, std=0.5,
                      spare_pages=4, num_layers=1, layer_idx=0, page_pad=0) -> Case:
    """Block-sparse top-k inputs ("Struct_msa_attention_ragged_paged": d_indices [Hkv, rows, topk]).

    Per (kv head, row): the block holding the row's position plus topk-1 distinct
    uniformly drawn earlier blocks, in random order. Output is always bf16.
    """
    rng = np.random.default_rng(seed)
    cache_lengths = [int(x) for x in cache_lengths]
    batch = len(cache_lengths)
    rows = [1] * batch if rows is None else [int(x) for x in rows]
    tokens = [cache_lengths[b] + rows[b] for b in range(batch)]
    kv, _ = _make_cache(rng, dtype, 2, num_layers, page_size, num_kv_heads, head_dim, tokens,
                        spare_pages, page_pad, cache_lengths)
    off = _row_offsets(rows)
    total_q = int(off[-1])
    d_idx = np.zeros((num_kv_heads, total_q, topk), np.int32)
    for b in range(batch):
        for i in range(rows[b]):
            r = int(off[b]) + i
            pos = cache_lengths[b] + i
            last = pos // block_size
            for g in range(num_kv_heads):
                k = min(topk - 1, last)
                earlier = rng.choice(last, k, replace=False) if k > 0 else np.zeros(0, np.int64)
                ids = np.concatenate([earlier, [last]])
                if len(ids) < topk:   # fewer blocks exist than topk: repeat is not allowed, pad with `last`
                    raise ValueError("topk exceeds the number of blocks at position %d" % pos)
                d_idx[g, r] = rng.permutation(ids)
    _fill_cache(kv, seed, 1, std, [(0, t - 1) for t in tokens], layer_idx)
    q = _normal((total_q, num_kv_heads * group, head_dim), seed, 2, std, dtype)
    return Case("block_sparse", name, seed, dtype, "bf16", q, off, max(rows), kv, layer_idx,
                float(np.float32(scale)), d_indices=d_idx, block_size=block_size,
                meta={"group": group, "topk": topk})


# --------------------------------------------------------------------------- dense

def make_dense(*, name="dense", seed, rows, num_kv_heads, group, head_dim, dtype, out_dtype, causal=True,
               window=-1, scale, std=1.0) -> Case:
    """Dense ragged attention inputs without a KV cache ("RaggedFlashAttentionGPU"): q
    [total, Hkv*group, D], k and v [total, Hkv, D], N(0, std^2); rows per sequence."""
    rows = [int(x) for x in rows]
    off = _row_offsets(rows)
    total = int(off[-1])
    q = _normal((total, num_kv_heads * group, head_dim), seed, 2, std, dtype)
    k = _normal((total, num_kv_heads, head_dim), seed, 3, std, dtype)
    v = _normal((total, num_kv_heads, head_dim), seed, 4, std, dtype)
    return Case("dense", name, seed, dtype, out_dtype, q, off, max(rows), None, 0, float(np.float32(scale)),
                window=int(window), k=k, v=v, causal=bool(causal), meta={"group": group})


# --------------------------------------------------------------------------- latent

def make_latent(*, name="latent", seed, decode_positions, prefill_positions, prefill_rows,
                num_heads, head_dim, dtype, out_dtype, window, swa_page_size, comp_page_size,
                num_comp, comp_ratio, unused_frac, scale, std=1.0, spare_pages=1) -> Case:
    """Latent window + compressed + sink inputs ("latent_sparse_attention_ragged_paged").

    Sequences: one decode row at each of ``decode_positions``, then ``prefill_rows``
    rows starting at each of ``prefill_positions``. Window leaf: token-paged, one
    latent head; only positions some row's window reaches hold values. Compressed
    leaf: entry-paged, floor(pos_last / comp_ratio) entries per sequence. Each row
    lists ``num_comp`` distinct entries from [0, floor(pos / comp_ratio)) in random
    order, then each slot independently becomes -1 with probability ``unused_frac``.
    """
    rng = np.random.default_rng(seed)
    starts = [int(p) for p in decode_positions] + [int(p) for p in prefill_positions]
    rows = [1] * len(decode_positions) + [int(prefill_rows)] * len(prefill_positions)
    batch = len(starts)
    last = [starts[b] + rows[b] - 1 for b in range(batch)]
    off = _row_offsets(rows)
    total_q = int(off[-1])
    # window leaf: logical pages cover 0..last; only pages touching a window get a physical page
    swa_lp = [last[b] // swa_page_size + 1 for b in range(batch)]
    win_lo = [max(0, starts[b] - window + 1) for b in range(batch)]
    live = [list(range(win_lo[b] // swa_page_size, last[b] // swa_page_size + 1)) for b in range(batch)]
    n_live = [len(x) for x in live]
    lut_live, num_pages, spare_ids = _page_pool(rng, n_live, spare_pages, max(swa_lp))
    nan_page = int(spare_ids[0])
    swa_lut = np.full((batch, max(swa_lp)), nan_page, np.uint32)
    for b in range(batch):
        for k, lp in enumerate(live[b]):
            swa_lut[b, lp] = lut_live[b, k]
    packed = swa_page_size * head_dim
    swa = PagedCache(torch.empty(num_pages * packed, dtype=TORCH_DTYPE[dtype]), dtype, num_pages, 1, 1,
                     swa_page_size, 1, head_dim, -1, swa_lut, np.asarray(starts, np.uint32), max(starts))
    _fill_cache(swa, seed, 1, std, [(win_lo[b], last[b]) for b in range(batch)], 0)
    # compressed leaf
    n_ent = [last[b] // comp_ratio for b in range(batch)]
    comp, _ = _make_cache(rng, dtype, 1, 1, comp_page_size, 1, head_dim, n_ent, spare_pages, 0,
                          np.asarray(n_ent, np.uint32))
    _fill_cache(comp, seed, 3, std, [(0, n_ent[b] - 1) for b in range(batch)], 0)
    comp_idx = np.full((total_q, num_comp), -1, np.int32)
    for b in range(batch):
        for i in range(rows[b]):
            r = int(off[b]) + i
            avail = (starts[b] + i) // comp_ratio
            k = min(num_comp, avail)
            comp_idx[r, :k] = rng.choice(avail, k, replace=False)
            drop = rng.random(num_comp) < unused_frac
            comp_idx[r, drop] = -1
    q = _normal((total_q, num_heads, head_dim), seed, 2, std, dtype)
    sink = _normal((num_heads,), seed, 4, 1.0, "f32").numpy().astype(np.float32)
    return Case("latent", name, seed, dtype, out_dtype, q, off, max(rows), swa, 0,
                float(np.float32(scale)), comp=comp, window=window, comp_indices=comp_idx,
                attn_sink=sink, meta={"comp_ratio": comp_ratio})


# --------------------------------------------------------------------------- key compression

@dataclass
class CompressCase:
    """One key-compression call ("QSACompressKeysPaged" Tensor shapes): raw index keys
    in plane 0, kv head 0 of a paged indexer cache, block_keys [batch * max_blocks, D]."""
    name: str
    seed: int
    dtype: str                    # keys, gamma and block_keys
    freq_dtype: str
    kv: PagedCache                # planes 2, num_kv_heads 1
    layer_idx: int
    key_counts: np.ndarray        # [batch] int32 = cache_lengths + this step's rows
    max_blocks: int
    ratio: int
    rotary_dim: int
    eps: float
    gamma: torch.Tensor           # [D] of dtype
    freqs: torch.Tensor           # [positions, rotary_dim] of freq_dtype: (cos, sin) pairs
    max_prompt_length: int
    kind: str = "compress"
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.key_counts)

    @property
    def head_dim(self) -> int:
        return self.kv.head_dim

    def blocks_per_sequence(self) -> np.ndarray:
        """Complete groups of ``ratio`` raw keys per sequence, capped at max_blocks."""
        kc = np.maximum(self.key_counts.astype(np.int64), 0)
        return np.minimum(kc // self.ratio, self.max_blocks)


def rope_table(positions: int, rotary_dim: int, base: float = 10000.0, dtype: str = "f32") -> torch.Tensor:
    """Rotary input table [positions, rotary_dim]: row p holds the pairs
    (cos(p * w_i), sin(p * w_i)), w_i = base^(-2i / rotary_dim), i < rotary_dim / 2."""
    if rotary_dim == 0:
        return torch.zeros((positions, 0), dtype=TORCH_DTYPE[dtype])
    w = base ** (-np.arange(0, rotary_dim, 2, dtype=np.float64) / rotary_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * w[None, :]
    t = np.stack([np.cos(ang), np.sin(ang)], axis=-1).reshape(positions, rotary_dim)
    return torch.from_numpy(t).to(torch.float32).to(TORCH_DTYPE[dtype])


def make_compress(*, name="compress", seed, cache_lengths, rows, page_size, num_layers, layer_idx, head_dim,
                  dtype, freq_dtype="f32", ratio, rotary_dim, eps=1e-6, max_blocks=None, spare_pages=4,
                  page_pad=0, std=1.0, positions=None) -> CompressCase:
    """Key-compression inputs: sequence b holds key_counts[b] = cache_lengths[b] + rows[b]
    raw keys N(0, std^2) at positions 0.. of plane 0 of ``layer_idx``; plane 1, other
    layers, positions past key_counts and spare pages are NaN. gamma = 1 + N(0, 0.25^2).
    max_blocks defaults to ceil(max key_counts / ratio); the rotary table has
    ``positions`` rows (default max_blocks * ratio)."""
    rng = np.random.default_rng(seed)
    cl = [int(x) for x in cache_lengths]
    rows = [int(x) for x in rows]
    kc = np.asarray([c + r for c, r in zip(cl, rows)], np.int32)
    kv, _ = _make_cache(rng, dtype, 2, num_layers, page_size, 1, head_dim, [int(k) for k in kc],
                        spare_pages, page_pad, cl)
    _fill_cache(kv, seed, 1, std, [(0, int(k) - 1) for k in kc], layer_idx)
    nan_fill_(kv.pages_view()[:, 1])
    if max_blocks is None:
        max_blocks = max(1, -(-int(kc.max()) // ratio)) if len(kc) else 1
    gamma = (1.0 + 0.25 * _normal((head_dim,), seed, 3, 1.0, "f32")).to(TORCH_DTYPE[dtype])
    npos = max_blocks * ratio if positions is None else positions
    return CompressCase(name, seed, dtype, freq_dtype, kv, layer_idx, kc, int(max_blocks), int(ratio),
                        int(rotary_dim), float(np.float32(eps)), gamma, rope_table(npos, rotary_dim, dtype=freq_dtype),
                        max(rows) if rows else 0)


# --------------------------------------------------------------------------- block selection

@dataclass
class SelectCase:
    """One block-selection call: an index query per row, block keys [batch * max_blocks, D]
    at a per-sequence stride, top-k complete blocks into token_indices [total_q, W]."""
    name: str
    seed: int
    dtype: str
    q_index: torch.Tensor          # [total_q, D]
    block_keys: torch.Tensor       # [batch * max_blocks, D]
    input_row_offsets: np.ndarray  # [batch + 1] uint32
    cache_lengths: np.ndarray      # [batch] uint32
    max_blocks: int
    ratio: int
    topk: int
    W: int
    max_prompt_length: int
    kind: str = "select"
    meta: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return self.q_index.shape[0]

    @property
    def batch(self) -> int:
        return len(self.input_row_offsets) - 1

    def positions(self) -> np.ndarray:
        off = self.input_row_offsets.astype(np.int64)
        pos = np.empty(self.total_q, np.int64)
        for b in range(self.batch):
            pos[off[b]:off[b + 1]] = int(self.cache_lengths[b]) + np.arange(off[b + 1] - off[b])
        return pos

    def candidates(self) -> np.ndarray:
        """Complete blocks each row may choose from."""
        return np.minimum((self.positions() + 1) // self.ratio, self.max_blocks)


def make_select(*, name="select", seed, rows, cache_lengths, head_dim, dtype, ratio, topk, W=None,
                max_blocks=None, integer=False) -> SelectCase:
    """Block-selection inputs: index queries and block keys N(0, 1) in ``dtype`` (or, with
    ``integer``, whole numbers in [-2, 2], whose dot products are exact in fp32, so equal
    scores are frequent and the tie rule is exercised). Block rows past a sequence's
    complete blocks are NaN. W defaults to topk * ratio + ratio - 1."""
    rng = np.random.default_rng(seed)
    rows = [int(x) for x in rows]
    cl = np.asarray([int(x) for x in cache_lengths], np.uint32)
    off = _row_offsets(rows)
    total_q = int(off[-1])
    keys_per_seq = [int(c) + r for c, r in zip(cl, rows)]
    if max_blocks is None:
        max_blocks = max(1, max(k // ratio for k in keys_per_seq)) if rows else 1
    batch = len(rows)
    if integer:
        q = torch.from_numpy(rng.integers(-2, 3, size=(total_q, head_dim)).astype(np.float32))
        bk = torch.from_numpy(rng.integers(-2, 3, size=(batch * max_blocks, head_dim)).astype(np.float32))
        q, bk = q.to(TORCH_DTYPE[dtype]), bk.to(TORCH_DTYPE[dtype])
    else:
        q = _normal((total_q, head_dim), seed, 4, 1.0, dtype)
        bk = _normal((batch * max_blocks, head_dim), seed, 5, 1.0, dtype)
    bkv = bk.view(batch, max_blocks, head_dim)
    for b in range(batch):
        nb = min(keys_per_seq[b] // ratio, max_blocks)
        nan_fill_(bkv[b, nb:])
    if W is None:
        W = topk * ratio + ratio - 1
    return SelectCase(name, seed, dtype, q, bk, off, cl, int(max_blocks), int(ratio), int(topk), int(W),
                      max(rows) if rows else 0, meta={"integer": integer})


# --------------------------------------------------------------------------- named workloads

def c1_tiny_fp32(seed=1):
    """Tiny fp32 sparse GQA: batch 2, rows [3,5], cache lengths [29,59], page 16, group 4, D 64."""
    return make_qsa(name="c1_tiny_fp32", seed=seed, rows=[3, 5], cache_lengths=[29, 59], page_size=16,
                    num_layers=1, layer_idx=0, num_kv_heads=1, group=4, head_dim=64, dtype="f32",
                    out_dtype="f32", selection_width=16, selection="uniform_counts", scale=1 / 8,
                    spare_pages=4)


def c2_decode_bf16(seed=2, batch=64):
    """bf16 decode: 64 rows, cache lengths U[1024,8192], page 128, 4 layers (layer 2),
    32 q heads / 8 kv heads, D 128, W 2048, counts = min(2048, pos+1)."""
    rng = np.random.default_rng(seed + 10_000)
    cl = rng.integers(1024, 8192, size=batch, endpoint=True)
    return make_qsa(name="c2_decode_bf16", seed=seed, rows=[1] * batch, cache_lengths=cl, page_size=128,
                    num_layers=4, layer_idx=2, num_kv_heads=8, group=4, head_dim=128, dtype="bf16",
                    out_dtype="bf16", selection_width=2048, selection="min", scale=1 / math.sqrt(128))


def c3_prefill_bf16(seed=3, batch=8, rows_range=(256, 2048), cache_range=(0, 4096)):
    """bf16 ragged prefill, group 16: rows U[256,2048], cache lengths U[0,4096], page 128,
    64 q heads / 4 kv heads, D 128, W 512 (last 64 positions + uniform earlier)."""
    rng = np.random.default_rng(seed + 10_000)
    rows = rng.integers(rows_range[0], rows_range[1], size=batch, endpoint=True)
    cl = rng.integers(cache_range[0], cache_range[1], size=batch, endpoint=True)
    return make_qsa(name="c3_prefill_bf16", seed=seed, rows=rows, cache_lengths=cl, page_size=128,
                    num_layers=1, layer_idx=0, num_kv_heads=4, group=16, head_dim=128, dtype="bf16",
                    out_dtype="bf16", selection_width=512, selection="recent", scale=1 / math.sqrt(128))


def c4_block_sparse_fp8(seed=4, batch=32, cache_range=(16384, 32768)):
    """Block-sparse top-16 of 64-token blocks, e4m3 q/KV, bf16 out: decode batch 32,
    cache lengths U[16k,32k], page 128, 32 q heads / 4 kv heads, D 128, values N(0, 0.5^2)."""
    rng = np.random.default_rng(seed + 10_000)
    cl = rng.integers(cache_range[0], cache_range[1], size=batch, endpoint=True)
    return make_block_sparse(name="c4_block_sparse_fp8", seed=seed, cache_lengths=cl, page_size=128,
                             num_kv_heads=4, group=8, head_dim=128, dtype="e4m3", topk=16,
                             block_size=64, scale=1 / math.sqrt(128), std=0.5)


def c4s_block_sparse_spec_fp8(seed=6, batch=32, draft=3, cache_range=(16384, 32768)):
    """Block-sparse speculative decode: the C4 shapes with `draft` query tokens per
    sequence, each at its own position (cache length + its index) with its own top-16
    blocks and its own causal clip."""
    rng = np.random.default_rng(seed + 10_000)
    cl = rng.integers(cache_range[0], cache_range[1], size=batch, endpoint=True)
    return make_block_sparse(name="c4s_block_sparse_spec_fp8", seed=seed, cache_lengths=cl, rows=[draft] * batch,
                             page_size=128, num_kv_heads=4, group=8, head_dim=128, dtype="e4m3", topk=16,
                             block_size=64, scale=1 / math.sqrt(128), std=0.5)


def c4p_block_sparse_prefill_bf16(seed=7, batch=4, rows=96, cache_range=(4096, 16384)):
    """Block-sparse prefill: `rows` new tokens per sequence (more than four: the pages'
    prefill case), bf16, 32 q heads / 4 kv heads, top-16 of 64-token blocks."""
    rng = np.random.default_rng(seed + 10_000)
    cl = rng.integers(cache_range[0], cache_range[1], size=batch, endpoint=True)
    return make_block_sparse(name="c4p_block_sparse_prefill_bf16", seed=seed, cache_lengths=cl, rows=[rows] * batch,
                             page_size=128, num_kv_heads=4, group=8, head_dim=128, dtype="bf16", topk=16,
                             block_size=64, scale=1 / math.sqrt(128), std=0.5)


def f3_dense_prefill_bf16(seed=8, batch=8, rows_range=(256, 2048)):
    """Dense causal ragged attention at the C3 prefill shapes (no cache): rows
    U[256, 2048] per sequence, 64 q heads / 4 kv heads, D 128, bf16; the sparse-vs-dense
    comparison at equal shapes."""
    rng = np.random.default_rng(3 + 10_000)          # C3's row draw
    rows = rng.integers(rows_range[0], rows_range[1], size=batch, endpoint=True)
    return make_dense(name="f3_dense_prefill_bf16", seed=seed, rows=rows, num_kv_heads=4, group=16,
                      head_dim=128, dtype="bf16", out_dtype="bf16", causal=True, window=-1,
                      scale=1 / math.sqrt(128))


def c5_latent_bf16(seed=5, n_decode=16, n_prefill=4, prefill_rows=128, pos_range=(2048, 65536)):
    """Latent window + compressed + sink: one latent head, D 512, 64 q heads, bf16;
    16 decode rows + 4 x 128 prefill rows, positions U[2k,64k], window 128 (page 64),
    512 compressed entries per row of pos/4, ~10% unused, per-head sink."""
    rng = np.random.default_rng(seed + 10_000)
    pos = rng.integers(pos_range[0], pos_range[1], size=n_decode + n_prefill, endpoint=True)
    return make_latent(name="c5_latent_bf16", seed=seed, decode_positions=pos[:n_decode],
                       prefill_positions=pos[n_decode:], prefill_rows=prefill_rows, num_heads=64,
                       head_dim=512, dtype="bf16", out_dtype="bf16", window=128, swa_page_size=64,
                       comp_page_size=64, num_comp=512, comp_ratio=4, unused_frac=0.1,
                       scale=1 / math.sqrt(512))


def f2_compress_keys_bf16(seed=9, batch=32, cache_range=(16384, 32768)):
    """Indexer key compression at the C4 decode shapes: 32 sequences, cache lengths
    U[16k, 32k] plus one new row each, D 128, bf16 keys / gamma / block keys, ratio 4,
    64 rotary channels from an fp32 table, page 128, 2 layers (layer 1)."""
    rng = np.random.default_rng(seed + 10_000)
    cl = rng.integers(cache_range[0], cache_range[1], size=batch, endpoint=True)
    return make_compress(name="f2_compress_keys_bf16", seed=seed, cache_lengths=cl, rows=[1] * batch,
                         page_size=128, num_layers=2, layer_idx=1, head_dim=128, dtype="bf16", freq_dtype="f32",
                         ratio=4, rotary_dim=64, eps=1e-6)


def f4_select_blocks_bf16(seed=10, batch=32, cache_range=(16384, 32768), topk=511):
    """Block selection at the indexer workload's shapes: one decode row per sequence
    (cache lengths U[16k, 32k]), blocks of 4 positions (4k-8k candidates per row), one
    bf16 index query of 128 channels per row, top 511 blocks into 511 * 4 + 3 = 2047
    positions."""
    rng = np.random.default_rng(seed + 10_000)
    cl = rng.integers(cache_range[0], cache_range[1], size=batch, endpoint=True)
    return make_select(name="f4_select_blocks_bf16", seed=seed, rows=[1] * batch, cache_lengths=cl, head_dim=128,
                       dtype="bf16", ratio=4, topk=topk)


NAMED = {
    "c1_tiny_fp32": c1_tiny_fp32,
    "c2_decode_bf16": c2_decode_bf16,
    "c3_prefill_bf16": c3_prefill_bf16,
    "c4_block_sparse_fp8": c4_block_sparse_fp8,
    "c4s_block_sparse_spec_fp8": c4s_block_sparse_spec_fp8,
    "c4p_block_sparse_prefill_bf16": c4p_block_sparse_prefill_bf16,
    "c5_latent_bf16": c5_latent_bf16,
    "f3_dense_prefill_bf16": f3_dense_prefill_bf16,
    "f2_compress_keys_bf16": f2_compress_keys_bf16,
    "f4_select_blocks_bf16": f4_select_blocks_bf16,
}


def gathered_kv_bytes(case: Case) -> int:
    """Algorithmic K/V bytes one call must gather (selected keys only).

    qsa: sum_r min(counts_r, W) * Hkv * 2 * D * elem; block-sparse: per (kv head, row)
    the listed block keys at or before the row's position; latent: window keys plus
    listed (>= 0) compressed entries, one latent row each.
    """
    eb = ELEM_BYTES[case.dtype]
    D = case.head_dim
    if case.kind == "qsa":
        W = case.token_indices.shape[1]
        n = np.clip(case.counts.astype(np.int64), 0, W).sum()
        return int(n) * case.kv.num_kv_heads * 2 * D * eb
    if case.kind == "dense":
        return int(dense_key_counts(case).sum()) * case.k.shape[1] * 2 * D * eb
    pos = case.positions()
    if case.kind == "block_sparse":
        bs = case.block_size
        ids = case.d_indices.astype(np.int64)                 # [Hkv, rows, topk]
        first = ids * bs
        nkeys = np.clip(pos[None, :, None] - first + 1, 0, bs).sum()
        return int(nkeys) * 2 * D * eb
    if case.kind == "latent":
        win = np.minimum(pos + 1, case.window).sum()
        comp = (case.comp_indices >= 0).sum()
        return int(win + comp) * D * eb
    raise ValueError(case.kind)


def compress_bytes(case: CompressCase) -> int:
    """Algorithmic bytes of one key-compression call: the raw keys of every complete
    group, the block keys written, each rotary table row used once (rows are shared
    across sequences), gamma, the key counts and the page-table entries read."""
    eb = ELEM_BYTES[case.dtype]
    D = case.head_dim
    nb = case.blocks_per_sequence()
    keys = int(nb.sum()) * case.ratio * D * eb
    writes = int(nb.sum()) * D * eb
    freqs = (int(nb.max()) if len(nb) else 0) * case.rotary_dim * ELEM_BYTES[case.freq_dtype]
    pages = int(sum(-(-int(n) * case.ratio // case.kv.page_size) for n in nb)) * 4
    return keys + writes + freqs + D * eb + 4 * case.batch + pages


def dense_key_counts(case: Case) -> np.ndarray:
    """Keys each row of a dense case attends to (its own sequence only): [lo, hi] with
    hi = i (causal) or L - 1, lo = max(0, i - window + 1) when window > 0."""
    off = case.input_row_offsets.astype(np.int64)
    n = np.empty(case.total_q, np.int64)
    for b in range(case.batch):
        L = off[b + 1] - off[b]
        i = np.arange(L)
        hi = i if case.causal else np.full(L, L - 1)
        lo = np.maximum(0, i - case.window + 1) if case.window > 0 else np.zeros(L, np.int64)
        n[off[b]:off[b + 1]] = hi - lo + 1
    return n
