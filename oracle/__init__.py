"""fp64 CPU oracle for index-selected sparse attention over a paged KV cache (and for
dense ragged attention without a cache, the comparison row, for the key
compression that produces the block keys, and for the top-k block selection that
turns them into token indices).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product library
never routes through it, and it shares no code with the HIP path.

The arithmetic lives in ``qsa_oracle.c`` (plain C, double precision, the plain
definition of each operation; see its header for the pages and sections each
function follows and the readings taken where the pages are silent). This module
only marshals numpy / torch-CPU arrays into it.

Every function is pinned by ``tests/test_oracle_pins.py``; none is "parity
unpinned" except where that file says so (the GQA head-to-kv-head mapping and the
latent key-equals-value reading are conventions that no page value fixes; so are the
key-compression choices of pooling operator, step order, rotation pairing and
rotation position, and the whole contract of block selection, which the pins check
as stated but the pages do not fix).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1, "e4m3": 2}


def compile_source(src: str, out: str) -> str:
    """gcc build of an oracle source file (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``qsa_oracle.c`` into ``liboracle.so`` next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


_libs = {}


def load(path: str = None):
    """ctypes handle of the oracle library (the default build, or another build at ``path``)."""
    if path is None:
        build(force=False)
        path = _LIB
    if path not in _libs:
        lib = ctypes.CDLL(path)
        P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.orc_decode.argtypes = [I, P, P, I64]
        lib.orc_qsa.argtypes = [P, P, I64, P, I, I64, I64, I64, P, I64,
                                P, I64, I64, I64, I64, I64, P, P, I64, I64,
                                P, I64, P, F, I]
        lib.orc_block_sparse.argtypes = [P, P, I64, P, I, I64, I64, I64, P, I64,
                                         P, I64, I64, I64, I64, I64, P, P, I64, I64,
                                         P, I64, I64, F, I]
        lib.orc_latent.argtypes = [P, P, I64, P, I, I64, I64, I64, P, I64,
                                   P, I64, I64, I64, I64, P, P, I64,
                                   P, I64, I64, I64, I64, P, I64,
                                   I64, I64, P, I64, P, F, I]
        lib.orc_dense.argtypes = [P, P, I64, P, P, P, I, I64, I64, I64, I64, P, I64, I, I64, F, I]
        lib.orc_compress.argtypes = [P, P, I, I64, I64, I64, I64, I64, I64, P, I64, I64, P, I64, I64, I64,
                                     P, P, I, I64, I64, F, I]
        lib.orc_select.argtypes = [P, P, P, P, P, I, I64, I64, P, P, I64, I64, I64, I64, I64, I]
        for f in (lib.orc_decode, lib.orc_qsa, lib.orc_block_sparse, lib.orc_latent, lib.orc_dense,
                  lib.orc_compress, lib.orc_select):
            f.restype = I
        _libs[path] = lib
    return _libs[path]


def default_threads() -> int:
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


class _Keep:
    """Holds contiguous host buffers alive for the duration of one oracle call."""

    def __init__(self):
        self.items = []

    def ptr(self, a):
        if a is None:
            return None
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            self.items.append(a)
            return a.data_ptr()
        a = np.ascontiguousarray(a)
        self.items.append(a)
        return a.ctypes.data


def _rows_arg(keep, rows, total_q):
    if rows is None:
        return None, total_q
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return keep.ptr(r), len(r)


def decode(dtype: str, raw, lib=None) -> np.ndarray:
    """Decode stored elements (f32 / bf16 / e4m3 bytes) exactly to float64."""
    lib = lib or load()
    keep = _Keep()
    if isinstance(raw, torch.Tensor):
        n = raw.numel()
    else:
        n = np.asarray(raw).size
    out = np.empty(n, np.float64)
    rc = lib.orc_decode(DT[dtype], keep.ptr(raw), out.ctypes.data, n)
    if rc:
        raise ValueError("orc_decode failed (%d)" % rc)
    return out


def _check(rc, what):
    if rc == 1:
        raise ValueError(what + ": input outside its contract (index, page id or shape)")
    if rc:
        raise MemoryError(what + ": out of memory")


def sparse_attention(*, q, dtype, input_row_offsets, kv_blocks, num_pages, num_layers, page_size,
                     num_kv_heads, page_stride, cache_lengths, kv_lookup_table, layer_idx,
                     token_indices, counts, scale, rows=None, nthreads=None, lib=None) -> np.ndarray:
    """Index-selected sparse GQA ("QSASparseAttentionRaggedPaged"); fp64 [n_rows, Hq, D]."""
    lib = lib or load()
    keep = _Keep()
    total_q, Hq, D = q.shape
    rp, n = _rows_arg(keep, rows, total_q)
    out = np.empty((n, Hq, D), np.float64)
    lut = np.asarray(kv_lookup_table, np.uint32)
    idx = np.asarray(token_indices, np.int32)
    rc = lib.orc_qsa(out.ctypes.data, rp, n, keep.ptr(q), DT[dtype], total_q, Hq, D,
                     keep.ptr(np.asarray(input_row_offsets, np.uint32)), len(input_row_offsets) - 1,
                     keep.ptr(kv_blocks), num_pages, num_layers, page_size, num_kv_heads, page_stride,
                     keep.ptr(np.asarray(cache_lengths, np.uint32)), keep.ptr(lut), lut.shape[1],
                     layer_idx, keep.ptr(idx), idx.shape[1], keep.ptr(np.asarray(counts, np.int32)),
                     scale, nthreads or default_threads())
    _check(rc, "orc_qsa")
    return out


def block_sparse_attention(*, q, dtype, input_row_offsets, kv_blocks, num_pages, num_layers,
                           page_size, num_kv_heads, page_stride, cache_lengths, kv_lookup_table,
                           layer_idx, d_indices, block_size, scale, rows=None,
                           nthreads=None, lib=None) -> np.ndarray:
    """Block-sparse top-k attention ("Struct_msa_attention_ragged_paged"); fp64 [n_rows, Hq, D]."""
    lib = lib or load()
    keep = _Keep()
    total_q, Hq, D = q.shape
    rp, n = _rows_arg(keep, rows, total_q)
    out = np.empty((n, Hq, D), np.float64)
    lut = np.asarray(kv_lookup_table, np.uint32)
    di = np.asarray(d_indices, np.int32)
    rc = lib.orc_block_sparse(out.ctypes.data, rp, n, keep.ptr(q), DT[dtype], total_q, Hq, D,
                              keep.ptr(np.asarray(input_row_offsets, np.uint32)),
                              len(input_row_offsets) - 1, keep.ptr(kv_blocks), num_pages, num_layers,
                              page_size, num_kv_heads, page_stride,
                              keep.ptr(np.asarray(cache_lengths, np.uint32)), keep.ptr(lut), lut.shape[1],
                              layer_idx, keep.ptr(di), di.shape[2], block_size, scale,
                              nthreads or default_threads())
    _check(rc, "orc_block_sparse")
    return out


def latent_sparse_attention(*, q, dtype, input_row_offsets, swa, comp, layer_idx, window,
                            comp_indices, attn_sink, scale, rows=None, nthreads=None, lib=None) -> np.ndarray:
    """Latent window + compressed + sink attention; fp64 [n_rows, Hq, D].

    ``swa`` and ``comp`` are dicts with blocks, num_pages, num_layers, page_size,
    page_stride, kv_lookup_table (and cache_lengths for ``swa``).
    """
    lib = lib or load()
    keep = _Keep()
    total_q, Hq, D = q.shape
    rp, n = _rows_arg(keep, rows, total_q)
    out = np.empty((n, Hq, D), np.float64)
    slut = np.asarray(swa["kv_lookup_table"], np.uint32)
    clut = np.asarray(comp["kv_lookup_table"], np.uint32)
    ci = np.asarray(comp_indices, np.int32)
    rc = lib.orc_latent(out.ctypes.data, rp, n, keep.ptr(q), DT[dtype], total_q, Hq, D,
                        keep.ptr(np.asarray(input_row_offsets, np.uint32)), len(input_row_offsets) - 1,
                        keep.ptr(swa["blocks"]), swa["num_pages"], swa["num_layers"], swa["page_size"],
                        swa["page_stride"], keep.ptr(np.asarray(swa["cache_lengths"], np.uint32)),
                        keep.ptr(slut), slut.shape[1],
                        keep.ptr(comp["blocks"]), comp["num_pages"], comp["num_layers"],
                        comp["page_size"], comp["page_stride"], keep.ptr(clut), clut.shape[1],
                        layer_idx, window, keep.ptr(ci), ci.shape[1],
                        keep.ptr(np.asarray(attn_sink, np.float32)), scale,
                        nthreads or default_threads())
    _check(rc, "orc_latent")
    return out


def dense_attention(*, q, k, v, dtype, input_row_offsets, causal, window, scale, rows=None,
                    nthreads=None, lib=None) -> np.ndarray:
    """Dense ragged attention without a KV cache ("RaggedFlashAttentionGPU"); fp64
    [n_rows, Hq, D]. k, v: [total_q, Hkv, D] of ``dtype``; window <= 0 means none."""
    lib = lib or load()
    keep = _Keep()
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    rp, n = _rows_arg(keep, rows, total_q)
    out = np.empty((n, Hq, D), np.float64)
    off = np.asarray(input_row_offsets, np.uint32)
    rc = lib.orc_dense(out.ctypes.data, rp, n, keep.ptr(q), keep.ptr(k), keep.ptr(v), DT[dtype], total_q, Hq,
                       Hkv, D, keep.ptr(off), len(off) - 1, int(bool(causal)), int(window), scale,
                       nthreads or default_threads())
    _check(rc, "orc_dense")
    return out


def compress_keys(*, kv_blocks, dtype, num_pages, num_planes, num_layers, page_size, head_dim, page_stride,
                  kv_lookup_table, layer_idx, key_counts, max_blocks, ratio, gamma, freqs_cis, freq_dtype,
                  rotary_dim, eps, nthreads=None, lib=None) -> np.ndarray:
    """Block keys pooled from raw index keys ("QSACompressKeysPaged"); fp64
    [batch * max_blocks, head_dim], NaN in the rows past each sequence's block count."""
    lib = lib or load()
    keep = _Keep()
    lut = np.asarray(kv_lookup_table, np.uint32)
    kc = np.asarray(key_counts, np.int32)
    batch = len(kc)
    out = np.empty((batch * max_blocks, head_dim), np.float64)
    npos = freqs_cis.shape[0]
    rc = lib.orc_compress(out.ctypes.data, keep.ptr(kv_blocks), DT[dtype], num_pages, num_planes, num_layers,
                          page_size, head_dim, page_stride, keep.ptr(lut), lut.shape[1], layer_idx, keep.ptr(kc),
                          batch, max_blocks, ratio, keep.ptr(gamma), keep.ptr(freqs_cis), DT[freq_dtype], npos,
                          rotary_dim, eps, nthreads or default_threads())
    _check(rc, "orc_compress")
    return out


def select_blocks(*, q_index, block_keys, dtype, input_row_offsets, cache_lengths, max_blocks, ratio, topk, W,
                  with_blocks=True, fill=-7, nthreads=None, lib=None):
    """Top-k block selection from block keys; returns (token_indices [total_q, W] int32 with
    ``fill`` past each row's count, counts [total_q] int32, blocks [total_q, topk] int32
    or None)."""
    lib = lib or load()
    keep = _Keep()
    total_q, D = q_index.shape
    off = np.asarray(input_row_offsets, np.uint32)
    idx = np.full((total_q, W), fill, np.int32)
    counts = np.zeros(total_q, np.int32)
    blocks = np.full((total_q, topk), -9, np.int32) if with_blocks else None
    rc = lib.orc_select(idx.ctypes.data, counts.ctypes.data, blocks.ctypes.data if with_blocks else None,
                        keep.ptr(q_index), keep.ptr(block_keys), DT[dtype], total_q, D, keep.ptr(off),
                        keep.ptr(np.asarray(cache_lengths, np.uint32)), len(off) - 1, max_blocks, ratio, topk, W,
                        nthreads or default_threads())
    _check(rc, "orc_select")
    return idx, counts, blocks


def _leaf(c):
    return dict(blocks=c.storage, num_pages=c.num_pages, num_layers=c.num_layers,
                page_size=c.page_size, num_kv_heads=c.num_kv_heads, page_stride=c.page_stride,
                kv_lookup_table=c.lookup_table, cache_lengths=c.cache_lengths)


def run_case(case, rows=None, nthreads=None, lib=None) -> np.ndarray:
    """Evaluate the oracle on a ``workloads.Case`` (all rows, or the listed ones)."""
    if case.kind == "qsa":
        kv = case.kv
        return sparse_attention(q=case.q, dtype=case.dtype, input_row_offsets=case.input_row_offsets,
                                kv_blocks=kv.storage, num_pages=kv.num_pages, num_layers=kv.num_layers,
                                page_size=kv.page_size, num_kv_heads=kv.num_kv_heads,
                                page_stride=kv.page_stride, cache_lengths=kv.cache_lengths,
                                kv_lookup_table=kv.lookup_table, layer_idx=case.layer_idx,
                                token_indices=case.token_indices, counts=case.counts,
                                scale=case.scale, rows=rows, nthreads=nthreads, lib=lib)
    if case.kind == "block_sparse":
        kv = case.kv
        return block_sparse_attention(q=case.q, dtype=case.dtype,
                                      input_row_offsets=case.input_row_offsets, kv_blocks=kv.storage,
                                      num_pages=kv.num_pages, num_layers=kv.num_layers,
                                      page_size=kv.page_size, num_kv_heads=kv.num_kv_heads,
                                      page_stride=kv.page_stride, cache_lengths=kv.cache_lengths,
                                      kv_lookup_table=kv.lookup_table, layer_idx=case.layer_idx,
                                      d_indices=case.d_indices, block_size=case.block_size,
                                      scale=case.scale, rows=rows, nthreads=nthreads, lib=lib)
    if case.kind == "latent":
        return latent_sparse_attention(q=case.q, dtype=case.dtype,
                                       input_row_offsets=case.input_row_offsets, swa=_leaf(case.kv),
                                       comp=_leaf(case.comp), layer_idx=case.layer_idx,
                                       window=case.window, comp_indices=case.comp_indices,
                                       attn_sink=case.attn_sink, scale=case.scale, rows=rows,
                                       nthreads=nthreads, lib=lib)
    if case.kind == "compress":
        kv = case.kv
        return compress_keys(kv_blocks=kv.storage, dtype=case.dtype, num_pages=kv.num_pages, num_planes=kv.planes,
                             num_layers=kv.num_layers, page_size=kv.page_size, head_dim=kv.head_dim,
                             page_stride=kv.page_stride, kv_lookup_table=kv.lookup_table,
                             layer_idx=case.layer_idx, key_counts=case.key_counts, max_blocks=case.max_blocks,
                             ratio=case.ratio, gamma=case.gamma, freqs_cis=case.freqs, freq_dtype=case.freq_dtype,
                             rotary_dim=case.rotary_dim, eps=case.eps, nthreads=nthreads, lib=lib)
    if case.kind == "select":
        return select_blocks(q_index=case.q_index, block_keys=case.block_keys, dtype=case.dtype,
                             input_row_offsets=case.input_row_offsets, cache_lengths=case.cache_lengths,
                             max_blocks=case.max_blocks, ratio=case.ratio, topk=case.topk, W=case.W,
                             nthreads=nthreads, lib=lib)
    if case.kind == "dense":
        return dense_attention(q=case.q, k=case.k, v=case.v, dtype=case.dtype,
                               input_row_offsets=case.input_row_offsets, causal=case.causal,
                               window=case.window, scale=case.scale, rows=rows, nthreads=nthreads, lib=lib)
    raise ValueError(case.kind)
