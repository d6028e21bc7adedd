"""Python binding of the MI355X sparse paged attention library (libqsa.so).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/qsa.h``. PyTorch supplies device memory and
the current stream. There is no fallback path: the import builds the library from
csrc/ when it is missing or out of date and fails if it cannot, and the functions
refuse CPU tensors.

Entry points (same names as the C ABI, without the ``qsa_`` prefix):

* ``sparse_attention`` - index-selected sparse GQA over a paged KV cache
  ("QSASparseAttentionRaggedPaged");
* ``block_sparse_attention`` - top-k KV blocks per (kv head, row), bf16 output
  ("Struct_msa_attention_ragged_paged");
* ``latent_sparse_attention`` - one latent head: sliding window + listed compressed
  entries + per-head sink ("latent_sparse_attention_ragged_paged");
* ``ragged_attention`` - dense ragged attention without a cache ("RaggedFlashAttentionGPU");
* ``compress_keys`` - block keys pooled from the raw index keys of a paged indexer
  cache ("QSACompressKeysPaged");
* ``select_blocks`` - top-k blocks per row from the block keys, as token_indices and
  counts for ``sparse_attention``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}
STATUS = {0: "QSA_OK", 1: "QSA_ERR_NULL", 2: "QSA_ERR_SHAPE", 3: "QSA_ERR_DTYPE",
          4: "QSA_ERR_UNSUPPORTED", 5: "QSA_ERR_WORKSPACE", 6: "QSA_ERR_HIP"}

# Every function declared in include/qsa.h.
EXPORTS = (
    "qsa_sparse_attention_workspace_size", "qsa_sparse_attention", "qsa_sparse_attention_no_alloc",
    "qsa_block_sparse_attention_workspace_size", "qsa_block_sparse_attention",
    "qsa_latent_sparse_attention_workspace_size", "qsa_latent_sparse_attention",
    "qsa_ragged_attention_workspace_size", "qsa_ragged_attention", "qsa_compress_keys",
    "qsa_select_blocks_workspace_size", "qsa_select_blocks",
    "qsa_last_error", "qsa_abi_version", "qsa_struct_size", "qsa_set_timing_events", "qsa_stream_read",
    "qsa_gather_replay",
)


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("num_planes", ctypes.c_int64),
                ("num_layers", ctypes.c_int64), ("page_size", ctypes.c_int64),
                ("num_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("page_stride", ctypes.c_int64), ("lookup_table", ctypes.c_void_p),
                ("max_pages", ctypes.c_int64), ("cache_lengths", ctypes.c_void_p),
                ("max_cache_length", ctypes.c_uint32), ("reserved1", ctypes.c_uint32)]


class _Ragged(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("num_q_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("batch", ctypes.c_int64),
                ("input_row_offsets", ctypes.c_void_p), ("max_prompt_length", ctypes.c_uint32),
                ("reserved1", ctypes.c_uint32)]


class LaunchOptions(ctypes.Structure):
    """Launch knobs: split-K partitions, wavefronts per workgroup, keys in flight (0 = auto)."""
    _fields_ = [("num_splits", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("unroll", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def _load():
    # libqsa.so is a build product (not kept in version control): build it from csrc/
    # when it is missing or was built from other sources. Without hipcc that fails
    # loudly; there is no other implementation to fall back to.
    from . import build as _build
    try:
        _build.ensure_built()
    except Exception as e:          # noqa: BLE001 - re-raised as the import failure it is
        raise ImportError("libqsa.so could not be built from %s: %s" % (_build.CSRC, e)) from e
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    pc, pr, po = ctypes.POINTER(_Cache), ctypes.POINTER(_Ragged), ctypes.POINTER(LaunchOptions)
    lib.qsa_sparse_attention_workspace_size.argtypes = [pr, pc, I64, po, ctypes.POINTER(SZ)]
    lib.qsa_sparse_attention.argtypes = [P, I32, pr, pc, ctypes.c_uint32, P, I64, P, F, po, P, SZ, P]
    lib.qsa_sparse_attention_no_alloc.argtypes = [P, I32, pr, pc, ctypes.c_uint32, P, I64, P, F, po, P]
    lib.qsa_block_sparse_attention_workspace_size.argtypes = [pr, pc, I64, I64, po, ctypes.POINTER(SZ)]
    lib.qsa_block_sparse_attention.argtypes = [P, pr, pc, ctypes.c_uint32, P, I64, I64, F, P, P, po,
                                               P, SZ, P]
    lib.qsa_latent_sparse_attention_workspace_size.argtypes = [pr, I64, I64, po, ctypes.POINTER(SZ)]
    lib.qsa_latent_sparse_attention.argtypes = [P, I32, pr, pc, pc, ctypes.c_uint32, I64, P, I64, P, F,
                                                po, P, SZ, P]
    lib.qsa_ragged_attention_workspace_size.argtypes = [pr, I64, I32, I64, po, ctypes.POINTER(SZ)]
    lib.qsa_ragged_attention.argtypes = [P, I32, pr, P, P, I64, I32, I64, F, po, P, SZ, P]
    U32 = ctypes.c_uint32
    lib.qsa_compress_keys.argtypes = [P, I64, P, P, I32, I64, I64, P, pc, I64, U32, U32, I64, F, P]
    lib.qsa_select_blocks_workspace_size.argtypes = [pr, I64, I64, I64, U32, ctypes.POINTER(SZ)]
    lib.qsa_select_blocks.argtypes = [P, I64, P, P, pr, P, I64, P, U32, I64, I64, P, SZ, P]
    for name in ("qsa_sparse_attention_workspace_size", "qsa_sparse_attention", "qsa_sparse_attention_no_alloc",
                 "qsa_block_sparse_attention_workspace_size", "qsa_block_sparse_attention",
                 "qsa_latent_sparse_attention_workspace_size", "qsa_latent_sparse_attention",
                 "qsa_ragged_attention_workspace_size", "qsa_ragged_attention", "qsa_compress_keys",
                 "qsa_select_blocks_workspace_size", "qsa_select_blocks"):
        getattr(lib, name).restype = ctypes.c_int
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_abi_version.restype = I32
    lib.qsa_struct_size.argtypes = [I32]
    lib.qsa_struct_size.restype = SZ
    lib.qsa_stream_read.argtypes = [P, SZ, P, U32, P]
    lib.qsa_stream_read.restype = ctypes.c_int
    lib.qsa_gather_replay.argtypes = [P, ctypes.c_uint64, P, P, U32, U32, U32, ctypes.c_int64, P, P]
    lib.qsa_gather_replay.restype = ctypes.c_int
    lib.qsa_set_timing_events.argtypes = [P, P]
    lib.qsa_set_timing_events.restype = None
    for i, st in enumerate((_Cache, _Ragged, LaunchOptions)):
        if lib.qsa_struct_size(i) != ctypes.sizeof(st):
            raise ImportError("ABI mismatch: %s is %d bytes in libqsa.so, %d here"
                              % (st.__name__, lib.qsa_struct_size(i), ctypes.sizeof(st)))
    return lib


lib = _load()


def _check(status: int):
    if status != 0:
        raise QsaError(status, lib.qsa_last_error().decode(errors="replace"))


@dataclass
class PagedCache:
    """Device view of one paged cache leaf (all tensors on the GPU).

    ``blocks`` holds [num_pages, num_planes, num_layers, page_size, num_kv_heads, head_dim]
    elements, pages ``page_stride`` elements apart (-1 = packed). ``lookup_table``
    [batch, max_pages] and ``cache_lengths`` [batch] are 32-bit integer tensors whose
    bits are read as uint32.
    """
    blocks: torch.Tensor
    num_pages: int
    num_planes: int
    num_layers: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    page_stride: int
    lookup_table: torch.Tensor
    cache_lengths: torch.Tensor
    max_cache_length: int = 0

    def _c(self) -> _Cache:
        _need_gpu(self.blocks, self.lookup_table, self.cache_lengths)
        _need_i32(self.lookup_table, self.cache_lengths)
        return _Cache(self.blocks.data_ptr(), DTYPE_CODE[self.blocks.dtype], 0, self.num_pages,
                      self.num_planes, self.num_layers, self.page_size, self.num_kv_heads,
                      self.head_dim, self.page_stride, self.lookup_table.data_ptr(),
                      self.lookup_table.shape[1], self.cache_lengths.data_ptr(),
                      self.max_cache_length, 0)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("sparse_attention_ragged_amd needs device tensors (got a CPU tensor)")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _need_i32(*ts):
    for t in ts:
        if t is not None and t.dtype not in (torch.int32, torch.uint32):
            raise ValueError("index tensors must be 32-bit integers, got %s" % t.dtype)


def _ragged(q: torch.Tensor, input_row_offsets: torch.Tensor, max_prompt_length: int) -> _Ragged:
    _need_gpu(q, input_row_offsets)
    _need_i32(input_row_offsets)
    if q.dim() != 3:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    return _Ragged(q.data_ptr(), DTYPE_CODE[q.dtype], 0, q.shape[0], q.shape[1], q.shape[2],
                   input_row_offsets.numel() - 1, input_row_offsets.data_ptr(), max_prompt_length, 0)


def _opts(options):
    if options is None:
        return None
    if isinstance(options, LaunchOptions):
        return ctypes.byref(options)
    unknown = set(options) - {"num_splits", "waves", "unroll"}
    if unknown:
        raise ValueError("unknown launch options: %s" % ", ".join(sorted(unknown)))
    o = LaunchOptions(options.get("num_splits", 0), options.get("waves", 0), options.get("unroll", 0), 0)
    return ctypes.byref(o)


def _stream(q: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small: %d bytes needed" % nbytes)
    return workspace, workspace.numel() * workspace.element_size()


def _out(q, out_dtype, out):
    if out is None:
        return torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need_gpu(out)
    if out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must be %s of %s" % (tuple(q.shape), out_dtype))
    return out


def sparse_attention_workspace_size(q, input_row_offsets, kv: PagedCache, selection_width: int,
                                    options=None, max_prompt_length: int = 0) -> int:
    n = ctypes.c_size_t(0)
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    ck = kv._c()
    _check(lib.qsa_sparse_attention_workspace_size(ctypes.byref(rq), ctypes.byref(ck), selection_width,
                                                   _opts(options), ctypes.byref(n)))
    return n.value


def sparse_attention(q, input_row_offsets, kv: PagedCache, layer_idx: int, token_indices, counts,
                     scale: float, *, out_dtype=None, max_prompt_length: int = 0, options=None,
                     out=None, workspace=None, stream=None) -> torch.Tensor:
    """Index-selected sparse GQA; returns out [total_q, num_q_heads, head_dim]."""
    out_dtype = out_dtype or (q.dtype if q.dtype != torch.float8_e4m3fn else torch.bfloat16)
    _need_gpu(token_indices, counts)
    _need_i32(token_indices, counts)
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    ck = kv._c()
    o = _opts(options)
    n = ctypes.c_size_t(0)
    W = token_indices.shape[1] if token_indices.dim() == 2 else 0
    _check(lib.qsa_sparse_attention_workspace_size(ctypes.byref(rq), ctypes.byref(ck), W, o,
                                                   ctypes.byref(n)))
    ws, wsb = _workspace(n.value, q.device, workspace)
    out = _out(q, out_dtype, out)
    _check(lib.qsa_sparse_attention(out.data_ptr(), DTYPE_CODE[out_dtype], ctypes.byref(rq),
                                    ctypes.byref(ck), layer_idx, token_indices.data_ptr(), W,
                                    counts.data_ptr(), scale, o,
                                    ws.data_ptr() if ws is not None else None, wsb, _stream(q, stream)))
    return out


NO_ALLOC_SCRATCH_BYTES = 16 << 20    # QSA_NO_ALLOC_SCRATCH_BYTES


def sparse_attention_no_alloc(q, input_row_offsets, kv: PagedCache, layer_idx: int, token_indices, counts,
                              scale: float, *, out, max_prompt_length: int = 0, options=None,
                              stream=None) -> torch.Tensor:
    """sparse_attention without a workspace: split-K partials go to the library's own
    device scratch (NO_ALLOC_SCRATCH_BYTES per GPU, shared by every such call on that
    GPU: calls that may overlap on one GPU race). ``out`` is required, so the call
    allocates nothing."""
    _need_gpu(token_indices, counts, out)
    _need_i32(token_indices, counts)
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    ck = kv._c()
    if out.shape != q.shape or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out must be %s of float32 or bfloat16" % (tuple(q.shape),))
    W = token_indices.shape[1] if token_indices.dim() == 2 else 0
    _check(lib.qsa_sparse_attention_no_alloc(out.data_ptr(), DTYPE_CODE[out.dtype], ctypes.byref(rq),
                                             ctypes.byref(ck), layer_idx, token_indices.data_ptr(), W,
                                             counts.data_ptr(), scale, _opts(options), _stream(q, stream)))
    return out


def block_sparse_attention_workspace_size(q, input_row_offsets, kv: PagedCache, topk: int,
                                          block_size: int, options=None) -> int:
    n = ctypes.c_size_t(0)
    rq = _ragged(q, input_row_offsets, 0)
    ck = kv._c()
    _check(lib.qsa_block_sparse_attention_workspace_size(ctypes.byref(rq), ctypes.byref(ck), topk,
                                                         block_size, _opts(options), ctypes.byref(n)))
    return n.value


def block_sparse_attention(q, input_row_offsets, kv: PagedCache, layer_idx: int, d_indices,
                           block_size: int, scale: float, *, max_prompt_length: int = 0,
                           cache_row_offsets=None, msa_scalar_args=None, options=None, out=None,
                           workspace=None, stream=None) -> torch.Tensor:
    """Block-sparse top-k attention; d_indices [num_kv_heads, total_q, topk]; bf16 output."""
    _need_gpu(d_indices, cache_row_offsets, msa_scalar_args)
    _need_i32(d_indices)
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    ck = kv._c()
    o = _opts(options)
    topk = d_indices.shape[2]
    n = ctypes.c_size_t(0)
    _check(lib.qsa_block_sparse_attention_workspace_size(ctypes.byref(rq), ctypes.byref(ck), topk,
                                                         block_size, o, ctypes.byref(n)))
    ws, wsb = _workspace(n.value, q.device, workspace)
    out = _out(q, torch.bfloat16, out)
    _check(lib.qsa_block_sparse_attention(
        out.data_ptr(), ctypes.byref(rq), ctypes.byref(ck), layer_idx, d_indices.data_ptr(), topk,
        block_size, scale, cache_row_offsets.data_ptr() if cache_row_offsets is not None else None,
        msa_scalar_args.data_ptr() if msa_scalar_args is not None else None, o,
        ws.data_ptr() if ws is not None else None, wsb, _stream(q, stream)))
    return out


def latent_sparse_attention_workspace_size(q, input_row_offsets, window: int, num_comp: int,
                                           options=None) -> int:
    n = ctypes.c_size_t(0)
    rq = _ragged(q, input_row_offsets, 0)
    _check(lib.qsa_latent_sparse_attention_workspace_size(ctypes.byref(rq), window, num_comp,
                                                          _opts(options), ctypes.byref(n)))
    return n.value


def latent_sparse_attention(q, input_row_offsets, swa: PagedCache, comp: PagedCache, layer_idx: int,
                            window: int, comp_indices, attn_sink, scale: float, *, out_dtype=None,
                            max_prompt_length: int = 0, options=None, out=None, workspace=None,
                            stream=None) -> torch.Tensor:
    """Latent window + compressed + sink attention; returns out [total_q, num_q_heads, head_dim]."""
    out_dtype = out_dtype or (q.dtype if q.dtype != torch.float8_e4m3fn else torch.bfloat16)
    _need_gpu(comp_indices, attn_sink)
    _need_i32(comp_indices)
    if attn_sink.dtype != torch.float32:
        raise ValueError("attn_sink must be float32")
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    cs, cc = swa._c(), comp._c()
    o = _opts(options)
    num_comp = comp_indices.shape[1]
    n = ctypes.c_size_t(0)
    _check(lib.qsa_latent_sparse_attention_workspace_size(ctypes.byref(rq), window, num_comp, o,
                                                          ctypes.byref(n)))
    ws, wsb = _workspace(n.value, q.device, workspace)
    out = _out(q, out_dtype, out)
    _check(lib.qsa_latent_sparse_attention(
        out.data_ptr(), DTYPE_CODE[out_dtype], ctypes.byref(rq), ctypes.byref(cs), ctypes.byref(cc),
        layer_idx, window, comp_indices.data_ptr(), num_comp, attn_sink.data_ptr(), scale, o,
        ws.data_ptr() if ws is not None else None, wsb, _stream(q, stream)))
    return out


def ragged_attention_workspace_size(q, input_row_offsets, num_kv_heads: int, causal: bool = True,
                                    window: int = -1, max_prompt_length: int = 0, options=None) -> int:
    n = ctypes.c_size_t(0)
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    _check(lib.qsa_ragged_attention_workspace_size(ctypes.byref(rq), num_kv_heads, int(bool(causal)), window,
                                                   _opts(options), ctypes.byref(n)))
    return n.value


def ragged_attention(q, k, v, input_row_offsets, scale: float, *, causal: bool = True, window: int = -1,
                     out_dtype=None, max_prompt_length: int, options=None, out=None, workspace=None,
                     stream=None) -> torch.Tensor:
    """Dense ragged attention without a KV cache; q [total, Hq, D], k/v [total, Hkv, D].
    max_prompt_length (host) must be at least the longest sequence. Returns out."""
    out_dtype = out_dtype or (q.dtype if q.dtype != torch.float8_e4m3fn else torch.bfloat16)
    _need_gpu(k, v)
    if k.dtype != q.dtype or v.dtype != q.dtype or k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must be [total, num_kv_heads, head_dim] of q's dtype")
    if k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("k and v must have q's rows and head_dim")
    if not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous")
    rq = _ragged(q, input_row_offsets, max_prompt_length)
    o = _opts(options)
    n = ctypes.c_size_t(0)
    _check(lib.qsa_ragged_attention_workspace_size(ctypes.byref(rq), k.shape[1], int(bool(causal)), window, o,
                                                   ctypes.byref(n)))
    ws, wsb = _workspace(n.value, q.device, workspace)
    out = _out(q, out_dtype, out)
    _check(lib.qsa_ragged_attention(
        out.data_ptr(), DTYPE_CODE[out_dtype], ctypes.byref(rq), k.data_ptr(), v.data_ptr(), k.shape[1],
        int(bool(causal)), window, scale, o, ws.data_ptr() if ws is not None else None, wsb, _stream(q, stream)))
    return out


def compress_keys(kv: PagedCache, key_counts, gamma, freqs_cis, layer_idx: int, ratio: int, rotary_dim: int,
                  eps: float, *, max_blocks: int, max_prompt_length: int = 0, out=None,
                  stream=None) -> torch.Tensor:
    """Block keys pooled from the raw index keys in plane 0 of ``kv``; key_counts [batch]
    int32; gamma [head_dim] of the cache dtype; freqs_cis [positions, rotary_dim] (float32
    or bfloat16 cos/sin pairs). Returns block_keys [batch * max_blocks, head_dim]; rows
    past a sequence's block count keep what ``out`` held (uninitialised when ``out`` is None)."""
    _need_gpu(key_counts, gamma, freqs_cis)
    _need_i32(key_counts)
    dt = kv.blocks.dtype
    if gamma.dtype != dt or gamma.numel() != kv.head_dim:
        raise ValueError("gamma must be [head_dim] of the cache dtype")
    if freqs_cis is not None and (freqs_cis.dim() != 2 or freqs_cis.shape[1] != rotary_dim):
        raise ValueError("freqs_cis must be [positions, rotary_dim]")
    batch = key_counts.numel()
    if batch != kv.lookup_table.shape[0]:
        raise ValueError("key_counts has %d sequences, the page table %d" % (batch, kv.lookup_table.shape[0]))
    shape = (batch * max_blocks, kv.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=kv.blocks.device)
    else:
        _need_gpu(out)
        if tuple(out.shape) != shape or out.dtype != dt:
            raise ValueError("out must be %s of %s" % (shape, dt))
    ck = kv._c()
    have_f = freqs_cis is not None and freqs_cis.numel() > 0
    _check(lib.qsa_compress_keys(out.data_ptr(), max_blocks, gamma.data_ptr(),
                                 freqs_cis.data_ptr() if have_f else None,
                                 DTYPE_CODE[freqs_cis.dtype] if freqs_cis is not None else F32,
                                 freqs_cis.shape[0] if freqs_cis is not None else 0, rotary_dim,
                                 key_counts.data_ptr(), ctypes.byref(ck), batch, layer_idx, max_prompt_length,
                                 ratio, eps, _stream(kv.blocks, stream)))
    return out


def stream_read(src: torch.Tensor, sink: torch.Tensor, grid: int = 2048, stream=None):
    """Plain streaming read of every byte of ``src`` (a calibration kernel, not an
    attention op); ``sink`` receives one int32 per workgroup (``grid`` of them)."""
    _need_gpu(src, sink)
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 4 * grid:
        raise ValueError("sink must hold %d 32-bit words" % grid)
    _check(lib.qsa_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), grid, _stream(src, stream)))


def gather_replay(base: torch.Tensor, offsets: torch.Tensor, counts: torch.Tensor, row_bytes: int,
                  plane_delta: int, sink: torch.Tensor, stream=None):
    """Bare replay of a recorded gather (a calibration kernel, not an attention op):
    item i reads the ``row_bytes`` rows at byte offsets ``offsets[i, :counts[i]]`` of
    ``base`` and the rows ``plane_delta`` bytes further on. ``offsets`` is int64
    [items, max_keys], ``counts`` int32 [items]; ``sink`` receives 256 int32 per item."""
    _need_gpu(base, offsets, counts, sink)
    if offsets.dtype != torch.int64 or offsets.dim() != 2 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int64 [items, max_keys] tensor")
    if counts.dtype != torch.int32 or counts.numel() != offsets.shape[0]:
        raise ValueError("counts must be int32 with one entry per item")
    items, max_keys = offsets.shape
    if sink.numel() * sink.element_size() < 4 * 256 * items:
        raise ValueError("sink must hold 256 32-bit words per item")
    _check(lib.qsa_gather_replay(base.data_ptr(), base.numel() * base.element_size(), offsets.data_ptr(),
                                 counts.data_ptr(), items, max_keys, row_bytes, plane_delta, sink.data_ptr(),
                                 _stream(base, stream)))


def select_blocks_workspace_size(q_index, input_row_offsets, max_blocks: int, ratio: int, topk: int,
                                 max_cache_length: int = 0, max_prompt_length: int = 0) -> int:
    n = ctypes.c_size_t(0)
    rq = _ragged(q_index.unsqueeze(1) if q_index.dim() == 2 else q_index, input_row_offsets, max_prompt_length)
    _check(lib.qsa_select_blocks_workspace_size(ctypes.byref(rq), max_blocks, ratio, topk, max_cache_length,
                                                ctypes.byref(n)))
    return n.value


def select_blocks(q_index, input_row_offsets, block_keys, cache_lengths, max_blocks: int, ratio: int, topk: int, *,
                  selection_width: int = 0, max_cache_length: int = 0, max_prompt_length: int = 0,
                  with_blocks: bool = True, token_indices=None, counts=None, blocks=None, workspace=None,
                  stream=None):
    """Top-k blocks per row from the block keys. q_index [total_q, head_dim] (one index
    query per row), block_keys [batch * max_blocks, head_dim] of the same dtype. Returns
    (token_indices [total_q, W] int32, counts [total_q] int32, blocks [total_q, topk] int32
    or None); W defaults to topk * ratio + ratio - 1. Entries of token_indices past a
    row's count keep what the tensor held (uninitialised when it is allocated here)."""
    q3 = q_index.unsqueeze(1) if q_index.dim() == 2 else q_index
    _need_gpu(q3, block_keys, cache_lengths, token_indices, counts, blocks)
    _need_i32(cache_lengths)
    if block_keys.dtype != q3.dtype or block_keys.dim() != 2 or block_keys.shape[1] != q3.shape[2]:
        raise ValueError("block_keys must be [batch * max_blocks, head_dim] of q_index's dtype")
    W = selection_width or topk * ratio + ratio - 1
    total_q, dev = q3.shape[0], q3.device
    rq = _ragged(q3, input_row_offsets, max_prompt_length)
    n = ctypes.c_size_t(0)
    _check(lib.qsa_select_blocks_workspace_size(ctypes.byref(rq), max_blocks, ratio, topk, max_cache_length,
                                                ctypes.byref(n)))
    if workspace is None and n.value > 0:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=dev)
    elif workspace is not None and workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small: %d bytes needed" % n.value)
    if token_indices is None:
        token_indices = torch.empty((total_q, W), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(total_q, dtype=torch.int32, device=dev)
    if blocks is None and with_blocks and topk > 0:
        blocks = torch.empty((total_q, topk), dtype=torch.int32, device=dev)
    if tuple(token_indices.shape) != (total_q, W) or counts.numel() != total_q:
        raise ValueError("token_indices must be [total_q, %d] and counts [total_q]" % W)
    _check(lib.qsa_select_blocks(token_indices.data_ptr(), W, counts.data_ptr(),
                                 blocks.data_ptr() if blocks is not None else None, ctypes.byref(rq),
                                 block_keys.data_ptr(), max_blocks, cache_lengths.data_ptr(), max_cache_length, ratio,
                                 topk, workspace.data_ptr() if workspace is not None else None,
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 _stream(q3, stream)))
    return token_indices, counts, blocks


def set_timing_events(start, stop) -> None:
    """Record two hipEvent_t handles (ints) around the main gather kernel of later calls
    on this thread; pass (None, None) to stop."""
    lib.qsa_set_timing_events(start, stop)
