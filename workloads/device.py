"""Move a generated ``Case`` to the GPU and call the library on it.

Input plumbing only (no arithmetic of the method): copies the host tensors of a
``workloads.Case`` to the device once and maps them onto the binding's argument
lists. The binding is imported lazily so that CPU-only users of ``workloads`` never
load the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


def _i32(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a.astype(np.int32, copy=False)).to(device)


def _leaf(c, device):
    import sparse_attention_ragged_amd as qsa
    return qsa.PagedCache(blocks=c.storage.to(device), num_pages=c.num_pages, num_planes=c.planes,
                          num_layers=c.num_layers, page_size=c.page_size, num_kv_heads=c.num_kv_heads,
                          head_dim=c.head_dim, page_stride=c.page_stride,
                          lookup_table=_i32(c.lookup_table, device),
                          cache_lengths=_i32(c.cache_lengths, device),
                          max_cache_length=int(c.max_cache_length))


@dataclass
class DeviceCase:
    case: object
    q: torch.Tensor
    row_off: torch.Tensor
    kv: object
    comp: Optional[object] = None
    token_indices: Optional[torch.Tensor] = None
    counts: Optional[torch.Tensor] = None
    d_indices: Optional[torch.Tensor] = None
    comp_indices: Optional[torch.Tensor] = None
    attn_sink: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None


def to_device(case, device="cuda") -> DeviceCase:
    dc = DeviceCase(case=case, q=case.q.to(device), row_off=_i32(case.input_row_offsets, device),
                    kv=_leaf(case.kv, device) if case.kv is not None else None)
    if case.kind == "dense":
        dc.k = case.k.to(device).contiguous()
        dc.v = case.v.to(device).contiguous()
    elif case.kind == "qsa":
        dc.token_indices = _i32(case.token_indices, device)
        dc.counts = _i32(case.counts, device)
    elif case.kind == "block_sparse":
        dc.d_indices = _i32(case.d_indices, device)
    else:
        dc.comp = _leaf(case.comp, device)
        dc.comp_indices = _i32(case.comp_indices, device)
        dc.attn_sink = torch.from_numpy(np.ascontiguousarray(case.attn_sink, np.float32)).to(device)
    return dc


def out_dtype(case) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[case.out_dtype]


def run(dc: DeviceCase, options=None, out=None, workspace=None, stream=None) -> torch.Tensor:
    """One library call on a device-resident case; returns the output tensor."""
    import sparse_attention_ragged_amd as qsa
    c = dc.case
    if c.kind == "qsa":
        return qsa.sparse_attention(dc.q, dc.row_off, dc.kv, c.layer_idx, dc.token_indices, dc.counts,
                                    c.scale, out_dtype=out_dtype(c), max_prompt_length=c.max_prompt_length,
                                    options=options, out=out, workspace=workspace, stream=stream)
    if c.kind == "dense":
        return qsa.ragged_attention(dc.q, dc.k, dc.v, dc.row_off, c.scale, causal=c.causal, window=c.window,
                                    out_dtype=out_dtype(c), max_prompt_length=c.max_prompt_length,
                                    options=options, out=out, workspace=workspace, stream=stream)
    if c.kind == "block_sparse":
        return qsa.block_sparse_attention(dc.q, dc.row_off, dc.kv, c.layer_idx, dc.d_indices,
                                          c.block_size, c.scale, max_prompt_length=c.max_prompt_length,
                                          options=options, out=out, workspace=workspace, stream=stream)
    return qsa.latent_sparse_attention(dc.q, dc.row_off, dc.kv, dc.comp, c.layer_idx, c.window,
                                       dc.comp_indices, dc.attn_sink, c.scale, out_dtype=out_dtype(c),
                                       max_prompt_length=c.max_prompt_length, options=options, out=out,
                                       workspace=workspace, stream=stream)


def workspace_size(dc: DeviceCase, options=None) -> int:
    import sparse_attention_ragged_amd as qsa
    c = dc.case
    if c.kind == "qsa":
        return qsa.sparse_attention_workspace_size(dc.q, dc.row_off, dc.kv, dc.token_indices.shape[1],
                                                   options)
    if c.kind == "dense":
        return qsa.ragged_attention_workspace_size(dc.q, dc.row_off, dc.k.shape[1], c.causal, c.window,
                                                   c.max_prompt_length, options)
    if c.kind == "block_sparse":
        return qsa.block_sparse_attention_workspace_size(dc.q, dc.row_off, dc.kv, dc.d_indices.shape[2],
                                                         c.block_size, options)
    return qsa.latent_sparse_attention_workspace_size(dc.q, dc.row_off, c.window,
                                                      dc.comp_indices.shape[1], options)


@dataclass
class DeviceCompress:
    case: object
    kv: object
    key_counts: torch.Tensor
    gamma: torch.Tensor
    freqs: torch.Tensor


def compress_to_device(case, device="cuda") -> DeviceCompress:
    """Device copies of a ``workloads.CompressCase``."""
    return DeviceCompress(case=case, kv=_leaf(case.kv, device), key_counts=_i32(case.key_counts, device),
                          gamma=case.gamma.to(device).contiguous(), freqs=case.freqs.to(device).contiguous())


def run_compress(dc: DeviceCompress, out=None, stream=None) -> torch.Tensor:
    """One key-compression call; returns block_keys [batch * max_blocks, head_dim]."""
    import sparse_attention_ragged_amd as qsa
    c = dc.case
    return qsa.compress_keys(dc.kv, dc.key_counts, dc.gamma, dc.freqs, c.layer_idx, c.ratio, c.rotary_dim, c.eps,
                             max_blocks=c.max_blocks, max_prompt_length=c.max_prompt_length, out=out,
                             stream=stream)


@dataclass
class DeviceSelect:
    case: object
    q_index: torch.Tensor
    block_keys: torch.Tensor
    row_off: torch.Tensor
    cache_lengths: torch.Tensor


def select_to_device(case, device="cuda") -> DeviceSelect:
    """Device copies of a ``workloads.SelectCase``."""
    return DeviceSelect(case=case, q_index=case.q_index.to(device).contiguous(),
                        block_keys=case.block_keys.to(device).contiguous(),
                        row_off=_i32(case.input_row_offsets, device), cache_lengths=_i32(case.cache_lengths, device))


def run_select(dc: DeviceSelect, token_indices=None, counts=None, blocks=None, workspace=None, stream=None):
    """One block-selection call; returns (token_indices, counts, blocks)."""
    import sparse_attention_ragged_amd as qsa
    c = dc.case
    return qsa.select_blocks(dc.q_index, dc.row_off, dc.block_keys, dc.cache_lengths, c.max_blocks, c.ratio, c.topk,
                             selection_width=c.W, max_cache_length=int(np.max(c.cache_lengths)) if c.batch else 0,
                             max_prompt_length=c.max_prompt_length, token_indices=token_indices, counts=counts,
                             blocks=blocks, workspace=workspace, stream=stream)
