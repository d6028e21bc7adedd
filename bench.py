#!/usr/bin/env python3
"""Benchmark: index-selected sparse GQA over a paged bf16 KV cache, decode shape.

Workload (one step = one call of qsa_sparse_attention = address generation + gather +
online softmax + split-K combine): 64 sequences with one query row each, cache
lengths U[1024, 8192], page size 128, 4 layers (layer 2 addressed), 32 q heads over
8 kv heads, head_dim 128, selection width 2048 with counts = min(2048, pos + 1),
bf16 in and out, synthetic seeded inputs (seed 2).

Inputs are resident in HBM before timing. To keep the timed steps honest about
caches, the KV pool is replicated R times at distinct addresses (R page tables
pointing at disjoint copies) and step k uses copy k mod R, so consecutive steps
never re-read what the previous one left in L2 or the 256 MiB MALL.

Prints one JSON line: throughput in gathered-KV GB/s (value), query rows/s, the
fraction of the 8 TB/s HBM peak, a roofline object for the gather kernel timed with
HIP events around that kernel alone, the fp64 CPU oracle timed on the host as a
baseline, and the same step measurements for the other workloads (ragged prefill
with 16 q heads per kv head, block-sparse e4m3 top-16 decode and speculative decode,
latent window + compressed + sink, dense causal prefill without a cache, the key
compression that produces the block keys, and the top-k block selection that turns
them into token indices) under "other_workloads".
"""
from __future__ import annotations

import argparse
import copy
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gathered-KV GB/s (% of HBM peak) + query-rows/s, bf16 decode config"
HBM_PEAK_GBPS = 8000.0
# the secondary workloads each follow seconds of host-side input generation: their
# warm-up runs until this much wall time has passed (the headline line keeps exactly
# --warmup calls, after the reference reads and pool copies that precede it)
OTHER_WARM_MS = 200.0


COUNTERS_SUMMARY = os.path.join(ROOT, "profiles", "gather_valu_c2_decode_bf16.md")


# The sources that build and plan the C2 gather kernel (its translation unit with the
# headers it includes, and the planner that picks its launch): the committed counter
# summary applies while these hash to the value stored with it.
GATHER_SOURCES = ("sparse_attention_ragged_amd/csrc/qsa_valu_bf16.hip",
                  "sparse_attention_ragged_amd/csrc/qsa_valu_kernel.hpp",
                  "sparse_attention_ragged_amd/csrc/qsa_valu_core.hpp",
                  "sparse_attention_ragged_amd/csrc/qsa_device.hpp", "sparse_attention_ragged_amd/csrc/qsa_host.hpp",
                  "sparse_attention_ragged_amd/csrc/qsa_plan.cpp", "include/qsa.h")

# Parity gates of the bench's own oracle checks (max abs, relative RMS) per element type.
PARITY_TOL = {"f32": (1e-4, 2e-6), "bf16": (2e-2, 1e-2), "e4m3": (6e-2, 1e-2)}


def _code_only(text):
    """C/C++ source without comments and whitespace: documentation edits leave the
    code (and so the kernel) unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


def csrc_digest():
    """sha256 over the gather kernel's sources (names and code without comments, in a
    fixed order)."""
    h = hashlib.sha256()
    for name in GATHER_SOURCES:
        h.update(name.encode())
        h.update(_code_only(open(os.path.join(ROOT, name), encoding="utf-8").read()).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gather kernel from the committed FETCH_SIZE/WRITE_SIZE
    summary, or None when there is none or the sources have changed since it was taken."""
    if not os.path.exists(COUNTERS_SUMMARY):
        return None
    fields = {}
    for line in open(COUNTERS_SUMMARY):
        k, sep, v = line.partition(":")
        if sep and k.strip() in ("traffic_bytes_per_launch", "csrc_sha256"):
            fields[k.strip()] = v.strip()
    if fields.get("csrc_sha256") != csrc_digest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs from the HIP runtime (the library records them on its stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0
            assert self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a.value, b.value))

    def ms(self, i):
        t = ctypes.c_float()
        a, b = self.pairs[i]
        rc = self.hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert rc == 0, rc
        return t.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(ctypes.c_void_p(a))
            self.hip.hipEventDestroy(ctypes.c_void_p(b))


def _replicate_leaf(leaf, R):
    import torch
    per = leaf.blocks.numel()
    big = torch.empty(per * R, dtype=leaf.blocks.dtype, device=leaf.blocks.device)
    reps = []
    for k in range(R):
        big[k * per:(k + 1) * per].copy_(leaf.blocks)
        c = copy.copy(leaf)
        c.blocks = big
        c.num_pages = leaf.num_pages * R
        c.lookup_table = (leaf.lookup_table.to(torch.int64) + k * leaf.num_pages).to(torch.int32).contiguous()
        reps.append(c)
    return reps


def replicate(dc, R):
    """R device cases whose KV pools (both pools for the latent workload) are copies at
    distinct addresses, each with its own page table."""
    kvs = _replicate_leaf(dc.kv, R)
    comps = _replicate_leaf(dc.comp, R) if dc.comp is not None else [None] * R
    out = []
    for k in range(R):
        c = copy.copy(dc)
        c.kv, c.comp = kvs[k], comps[k]
        out.append(c)
    return out


def algorithmic(case):
    """Per-launch algorithmic work of the gather kernel: gathered K/V bytes, the unit of
    work with its count and bytes (K/V rows plus the index that names them), and flops
    (Q.K^T plus P.V, 2 flops per multiply-add)."""
    import numpy as np
    import workloads as W
    eb = W.ELEM_BYTES[case.dtype]
    D, Hq = case.head_dim, case.num_q_heads
    gathered = W.gathered_kv_bytes(case)
    if case.kind == "qsa":
        units = int(np.clip(case.counts, 0, case.token_indices.shape[1]).sum())
        per_unit = case.kv.num_kv_heads * 2 * D * eb + 4
        flops = units * 4 * D * Hq
        unit = "(query row, selected key): Hkv*2*D*elem K/V bytes + 4 index bytes"
    elif case.kind == "block_sparse":
        units = gathered // (2 * D * eb)
        per_unit = 2 * D * eb
        flops = units * 4 * D * (Hq // case.kv.num_kv_heads)
        unit = "(query row, kv head, key in a listed block): 2*D*elem K/V bytes"
    elif case.kind == "dense":
        hkv = case.k.shape[1]
        units = int(W.dense_key_counts(case).sum())
        per_unit = hkv * 2 * D * eb
        flops = units * 4 * D * Hq
        unit = "(query row, key of its sequence): Hkv*2*D*elem K/V bytes"
    else:
        units = gathered // (D * eb)
        per_unit = D * eb
        flops = units * 4 * D * Hq
        unit = "(query row, window or compressed key): D*elem latent bytes"
    return dict(gathered=gathered, units=int(units), per_unit=per_unit, unit=unit,
                algo_bytes=int(units) * per_unit, flops=int(flops))


def prepare(case, R, dev, opts):
    """Device-resident inputs (R pool copies when R > 1), workspace and output."""
    import torch
    from workloads import device as D
    dc = D.to_device(case, dev)
    calls = replicate(dc, R) if R > 1 else [dc]
    del dc
    torch.cuda.synchronize()
    ws_n = D.workspace_size(calls[0], opts)
    ws = torch.zeros(max(ws_n, 16), dtype=torch.uint8, device=dev)   # zero-filled once
    out = torch.empty(tuple(case.q.shape), dtype=D.out_dtype(case), device=dev)
    return calls, ws, out


def time_steps(calls, opts, out, ws, stream, steps, warmup, warm_ms=0.0):
    """Milliseconds per step over `steps` back-to-back calls (step k uses calls[k % R]),
    then the gather kernel's average milliseconds from the HIP events the library
    records around it, over a second pass of `steps` calls."""
    from workloads import device as D
    R = len(calls)

    def step(k):
        D.run(calls[k % R], options=opts, out=out, workspace=ws, stream=stream)

    return time_step_fn(step, steps, warmup, warm_ms)


def time_step_fn(step, steps, warmup, warm_ms=0.0):
    """For any step(k) callable that makes one library call: milliseconds per step over
    `steps` back-to-back calls (wall clock between two synchronisations); then the
    main kernel's average from the HIP events the library records around it, over a
    second pass; then each call's own duration from events around the whole call
    (kernels and any combine step) over a third pass, as median, p10 and p90. With
    warm_ms > 0 the warm-up goes on (past `warmup` calls) until that much wall time has
    passed, so that a workload timed right after host-side input generation (the GPU
    idle, its clocks down) is not timed while the clocks ramp up."""
    import numpy as np
    import torch
    import sparse_attention_ragged_amd as qsa
    t_w = time.perf_counter()
    k = 0
    while k < warmup or (warm_ms > 0 and (time.perf_counter() - t_w) * 1e3 < warm_ms and k < 100000):
        step(k)
        k += 1
        if warm_ms > 0 and k % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    ev = HipEvents(steps)
    for k in range(steps):
        qsa.set_timing_events(*ev.pairs[k])
        step(k)
    torch.cuda.synchronize()
    qsa.set_timing_events(None, None)
    kern = sum(ev.ms(k) for k in range(steps)) / steps
    ev.close()
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        marks[k][0].record()
        step(k)
        marks[k][1].record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in marks])
    pct = {"median_us": round(float(np.median(per)) * 1e3, 2), "p10_us": round(float(np.percentile(per, 10)) * 1e3, 2),
           "p90_us": round(float(np.percentile(per, 90)) * 1e3, 2)}
    return ms_step, kern, pct


def parity(case, out, rows=None):
    """Max abs and relative RMS difference to the fp64 oracle (every row unless `rows`),
    and whether both are within the gates of the case's element type."""
    import numpy as np
    import oracle
    ref = oracle.run_case(case, rows=rows)
    got = (out if rows is None else out[list(rows)]).float().cpu().double().numpy()
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    rel = float(np.sqrt((err ** 2).mean()) / rms) if rms > 0 else 0.0
    tol, gate = PARITY_TOL["f32" if case.dtype == "f32" and case.out_dtype == "f32" else
                           ("e4m3" if case.dtype == "e4m3" else "bf16")]
    finite = bool(np.isfinite(got).all())
    return {"max_abs": max_abs, "rel_rms": rel, "rows_checked": int(ref.shape[0]),
            "ok": finite and max_abs <= tol and rel <= gate, "max_abs_tol": tol, "rel_rms_gate": gate}


def stream_read_reference(dev, stream, nbytes=4 << 30, reps=10):
    """GB/s of the library's plain streaming-read kernel over a buffer far larger than
    the caches, best over a few grid sizes: the practical read bandwidth of this GPU."""
    import torch
    import sparse_attention_ragged_amd as qsa
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    best = None
    for grid in (1024, 2048, 4096, 8192):
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        for _ in range(3):
            qsa.stream_read(buf, sink, grid=grid, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            qsa.stream_read(buf, sink, grid=grid, stream=stream)
        b.record()
        torch.cuda.synchronize()
        gbps = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, grid)
    del buf
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 1), "bytes": nbytes, "grid": best[1],
            "kernel": "qsa_stream_read: 16-byte nontemporal loads, 256-thread workgroups, 4 loads in flight per thread"}


def key_row_offsets(case):
    """Byte offsets, within the cache storage, of the K row (plane 0, the addressed layer)
    of every (row, kv head, selected key) of a token-index case, in the gather kernel's
    item order (row-major, kv head fastest); keys past a row's count are not listed."""
    import numpy as np
    kv = case.kv
    H, D, ps = kv.num_kv_heads, kv.head_dim, kv.page_size
    eb = 2 if case.dtype == "bf16" else (4 if case.dtype == "fp32" else 1)
    W = case.token_indices.shape[1]
    off = case.input_row_offsets.astype(np.int64)
    items = case.total_q * H
    offs = np.zeros((items, W), np.int64)
    counts = np.zeros(items, np.int32)
    for r in range(case.total_q):
        b = int(np.searchsorted(off, r, side="right") - 1)
        n = int(min(max(int(case.counts[r]), 0), W))
        toks = case.token_indices[r, :n].astype(np.int64)
        phys = kv.lookup_table[b][toks // ps].astype(np.int64)
        base = phys * kv.page_elems + case.layer_idx * ps * H * D + (toks % ps) * H * D
        for g in range(H):
            offs[r * H + g, :n] = (base + g * D) * eb
            counts[r * H + g] = n
    plane_delta = kv.num_layers * ps * H * D * eb
    return offs, counts, D * eb, plane_delta


def address_replay_reference(case, dc, dev, stream, reps=10):
    """Microseconds of the library's bare gather replay (qsa_gather_replay) over the
    exact K/V rows the gather kernel reads for this call (same pool, same rows, same
    workgroup per (row, kv head) and order), with no address computation or arithmetic:
    what this access pattern itself reaches on this GPU."""
    import numpy as np
    import torch
    import sparse_attention_ragged_amd as qsa
    offs, counts, row_bytes, plane_delta = key_row_offsets(case)
    d_offs = torch.from_numpy(offs).to(dev)
    d_counts = torch.from_numpy(counts).to(dev)
    sink = torch.empty(offs.shape[0] * 256, dtype=torch.int32, device=dev)
    base = dc.kv.blocks
    for _ in range(3):
        qsa.gather_replay(base, d_offs, d_counts, row_bytes, plane_delta, sink, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        qsa.gather_replay(base, d_offs, d_counts, row_bytes, plane_delta, sink, stream=stream)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    nbytes = int(counts.astype(np.int64).sum()) * 2 * row_bytes
    return {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "kv_bytes": nbytes,
            "kernel": "qsa_gather_replay: the recorded K/V row offsets of this call, one 256-thread "
                      "workgroup per (row, kv head), 16-byte non-temporal row-contiguous loads, two batches "
                      "in flight"}


def other_workload(name, make, R, dev, stream, steps, warmup):
    import torch
    log("%s: generating" % name)
    case = make()
    a = algorithmic(case)
    calls, ws, out = prepare(case, R, dev, None)
    log("%s: timing %d steps (+ %d with kernel events, + %d with step events)" % (name, steps, steps, steps))
    ms_step, kern, pct = time_steps(calls, None, out, ws, stream, steps, warmup, OTHER_WARM_MS)
    log("%s: parity on every row" % name)
    par = parity(case, out)
    res = {"workload": name, "query_rows": case.total_q, "dtype": case.dtype,
           "gathered_kv_bytes_per_step": a["gathered"], "kv_pool_replicas": R, "steps": steps,
           "ms_per_step": round(ms_step, 5), "step_events": pct,
           "gathered_GBps": round(a["gathered"] / (ms_step * 1e-3) / 1e9, 1),
           "query_rows_per_s": round(case.total_q / (ms_step * 1e-3), 1),
           "gather_kernel_avg_us": round(kern * 1e3, 2),
           "gather_kernel_GBps": round(a["algo_bytes"] / (kern * 1e-3) / 1e9, 1),
           "gather_kernel_TFLOPs": round(a["flops"] / (kern * 1e-3) / 1e12, 2),
           "unit_of_work": a["unit"], "units_per_launch": a["units"], "parity": par}
    del calls, ws, out
    torch.cuda.empty_cache()
    return res


def compress_workload(name, make, R, dev, stream, steps, warmup):
    """Key compression (the step that produces the block keys): raw index keys read once,
    block keys written once; the indexer pool is replicated R times."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    from workloads import device as D
    log("%s: generating" % name)
    case = make()
    dc = D.compress_to_device(case, dev)
    calls = []
    for leaf in _replicate_leaf(dc.kv, R):
        c = copy.copy(dc)
        c.kv = leaf
        calls.append(c)
    del dc
    out = torch.empty((case.batch * case.max_blocks, case.head_dim), dtype=W.TORCH_DTYPE[case.dtype], device=dev)
    torch.cuda.synchronize()
    log("%s: timing %d steps (+ %d with kernel events, + %d with step events)" % (name, steps, steps, steps))
    ms_step, kern, pct = time_step_fn(lambda k: D.run_compress(calls[k % R], out=out, stream=stream), steps, warmup,
                                      OTHER_WARM_MS)
    nb = case.blocks_per_sequence()
    algo = W.compress_bytes(case)
    ref = oracle.run_case(case)
    live = ~np.isnan(ref)
    got = out.float().cpu().double().numpy()
    res = {"workload": name, "sequences": case.batch, "block_keys": int(nb.sum()), "dtype": case.dtype,
           "raw_key_bytes_per_step": int(nb.sum()) * case.ratio * case.head_dim * W.ELEM_BYTES[case.dtype],
           "algorithmic_bytes_per_step": algo, "kv_pool_replicas": R, "steps": steps,
           "ms_per_step": round(ms_step, 5), "step_events": pct,
           "GBps": round(algo / (ms_step * 1e-3) / 1e9, 1),
           "compress_kernel_avg_us": round(kern * 1e3, 2),
           "compress_kernel_GBps": round(algo / (kern * 1e-3) / 1e9, 1),
           "unit_of_work": "block key: ratio*D*elem raw key bytes + D*elem written (+ table, gamma, counts, page entries)",
           "parity": {"max_abs_all_block_keys": float(np.abs(got[live] - ref[live]).max()),
                      "ok": bool(np.isfinite(got[live]).all() and np.abs(got[live] - ref[live]).max() <= 2e-2)}}
    del calls, out
    torch.cuda.empty_cache()
    return res


def select_workload(name, make, dev, stream, steps, warmup):
    """Top-k block selection (scores of every visible block key, then a radix top-k per
    row): block keys and queries read once per row; token indices, counts and block ids
    written."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    from workloads import device as D
    log("%s: generating" % name)
    case = make()
    dc = D.select_to_device(case, dev)
    idx = torch.empty((case.total_q, case.W), dtype=torch.int32, device=dev)
    counts = torch.empty(case.total_q, dtype=torch.int32, device=dev)
    blocks = torch.empty((case.total_q, case.topk), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log("%s: timing %d steps (+ %d with kernel events, + %d with step events)" % (name, steps, steps, steps))
    ms_step, kern, pct = time_step_fn(lambda k: D.run_select(dc, token_indices=idx, counts=counts, blocks=blocks,
                                                             stream=stream), steps, warmup, OTHER_WARM_MS)
    nv = case.candidates()
    eb = W.ELEM_BYTES[case.dtype]
    D_ = case.q_index.shape[1]
    cnt = counts.cpu().numpy()
    algo = int(nv.sum()) * D_ * eb + case.total_q * D_ * eb + int(cnt.sum()) * 4 + case.total_q * (4 + 4 * case.topk)
    ref = oracle.run_case(case)
    res = {"workload": name, "rows": case.total_q, "candidate_blocks": int(nv.sum()), "topk": case.topk,
           "dtype": case.dtype, "algorithmic_bytes_per_step": algo, "steps": steps,
           "ms_per_step": round(ms_step, 5), "step_events": pct, "select_kernels_avg_us": round(kern * 1e3, 2),
           "select_GBps": round(algo / (kern * 1e-3) / 1e9, 1),
           "rows_per_s": round(case.total_q / (ms_step * 1e-3), 1),
           "unit_of_work": "(row, candidate block): D*elem block-key bytes (+ the query, indices, counts, ids)",
           "parity": {"counts_match_oracle": bool(np.array_equal(cnt, ref[1])),
                      "ok": bool(np.array_equal(cnt, ref[1]))}}
    del dc, idx, counts, blocks
    torch.cuda.empty_cache()
    return res


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(case, threads, budget_s, min_reps=1):
    """Seconds per oracle call over the whole case, repeated for about budget_s."""
    import oracle
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.run_case(case, nthreads=threads)
        n += 1
        if n >= min_reps and time.perf_counter() - t0 >= budget_s:
            break
    return (time.perf_counter() - t0) / n, n


def cpu_baseline(case, budget_s):
    """The fp64 oracle on the host cores over the whole decode workload, repeated for
    about `budget_s` seconds (at least once), plus single-thread times of the tiny
    fp32, decode and block-sparse workloads."""
    import oracle
    import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    oracle.run_case(case, nthreads=threads)          # page in / build
    dt, n = _oracle_rate(case, threads, budget_s)
    gb = W.gathered_kv_bytes(case) / 1e9
    single = {}
    for name, c, budget in (("c1_tiny_fp32", W.c1_tiny_fp32(), 0.5), ("c2_decode_bf16", case, 3.0),
                            ("c4_block_sparse_fp8", W.c4_block_sparse_fp8(), 2.0)):
        t, reps = _oracle_rate(c, 1, budget)
        g = W.gathered_kv_bytes(c) / 1e9
        single[name] = {"s_per_call": round(t, 6), "reps": reps, "gathered_GBps": round(g / t, 4),
                        "query_rows_per_s": round(c.total_q / t, 2)}
    return {"value": round(gb / dt, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "whole c2_decode_bf16 workload (%d query rows, %.1f MB gathered K/V) x %d repetitions, "
                      "fp64 C oracle with OpenMP over (row, kv head); %.3f s per call, %.1f query-rows/s"
                      % (case.total_q, gb * 1e3, n, dt, case.total_q / dt),
            "threads": threads, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "cpu_model": _cpu_model(), "single_thread": single}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--unroll", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one of the other workloads alone (for profiling) and print its JSON object")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after warmup, run one device-to-device copy of this many MiB (a kernel "
                         "of known traffic for calibrating hardware byte counters)")
    ap.add_argument("--stream-probe-mib", type=int, default=0,
                    help="run one plain streaming read (qsa_stream_read) of this many MiB first: a "
                         "read-only kernel of known traffic for calibrating hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run "
              "the same kernel on its own shard of sequences or kv heads). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d bytes read, %d bytes written" % (src.numel(), dst.numel()))
        del src, dst
    if args.stream_probe_mib:
        import sparse_attention_ragged_amd as qsa
        src = torch.ones(args.stream_probe_mib << 20, dtype=torch.uint8, device=dev)
        sink = torch.empty(2048, dtype=torch.int32, device=dev)
        qsa.stream_read(src, sink, grid=2048, stream=stream)
        torch.cuda.synchronize()
        log("stream probe: %d bytes read" % src.numel())
        del src, sink
    n_other = max(5, min(args.steps, 20))
    others = {
        "c3_prefill_bf16": lambda: other_workload("c3_prefill_bf16", W.c3_prefill_bf16, 1, dev, stream, n_other, 3),
        "c4_block_sparse_fp8": lambda: other_workload("c4_block_sparse_fp8", W.c4_block_sparse_fp8, 8, dev, stream,
                                                      n_other, 3),
        "c4s_block_sparse_spec_fp8": lambda: other_workload("c4s_block_sparse_spec_fp8", W.c4s_block_sparse_spec_fp8,
                                                            8, dev, stream, n_other, 3),
        "c5_latent_bf16": lambda: other_workload("c5_latent_bf16", W.c5_latent_bf16, 4, dev, stream, n_other, 3),
        "f3_dense_prefill_bf16": lambda: other_workload("f3_dense_prefill_bf16", W.f3_dense_prefill_bf16, 1, dev,
                                                        stream, n_other, 3),
        "f2_compress_keys_bf16": lambda: compress_workload("f2_compress_keys_bf16", W.f2_compress_keys_bf16, 4, dev,
                                                          stream, n_other, 3),
        "f4_select_blocks_bf16": lambda: select_workload("f4_select_blocks_bf16", W.f4_select_blocks_bf16, dev,
                                                        stream, n_other, 3),
    }
    if args.only:
        if args.only not in others:
            print("unknown workload %s (one of %s)" % (args.only, ", ".join(others)), file=sys.stderr)
            sys.exit(2)
        print(json.dumps(others[args.only]()), flush=True)
        return
    log("stream-read reference")
    stream_ref = stream_read_reference(dev, stream)
    log("generating c2_decode_bf16 (seed 2)")
    case = W.c2_decode_bf16()
    a = algorithmic(case)
    gathered = a["gathered"]
    log("to device (%.2f GB pool x %d copies)" % (case.kv.storage.numel() * 2 / 1e9, args.replicas))
    opts = {"num_splits": args.splits, "waves": args.waves, "unroll": args.unroll}
    calls, ws, out = prepare(case, args.replicas, dev, opts)
    log("timing %d steps (+ %d with kernel events, + %d with step events)" % (args.steps, args.steps, args.steps))
    ms_step, kern_avg, pct = time_steps(calls, opts, out, ws, stream, args.steps, args.warmup)

    # parity of the last timed output on every row (the oracle takes well under a second)
    par = parity(case, out)
    log("address replay reference")
    replay = address_replay_reference(case, calls[0], dev, stream)

    value = gathered / (ms_step * 1e-3) / 1e9
    achieved = a["algo_bytes"] / (kern_avg * 1e-3) / 1e9
    traffic = measured_traffic()
    res = {
        "metric": METRIC,
        "value": round(value, 2) if par["ok"] else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c2_decode_bf16", "batch": case.batch, "query_rows": case.total_q,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.kv.num_kv_heads,
                   "head_dim": case.head_dim, "page_size": case.kv.page_size,
                   "num_layers": case.kv.num_layers, "layer_idx": case.layer_idx,
                   "selection_width": int(case.token_indices.shape[1]), "seed": case.seed,
                   "kv_pool_replicas": args.replicas, "launch": opts},
        "query_rows_per_s": round(case.total_q / (ms_step * 1e-3), 1),
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "stream_read_frac": round(value / stream_ref["GBps"], 4),
        "step_events": pct,
        "gathered_kv_bytes_per_step": gathered,
        "parity": par,
        "stream_read_reference": stream_ref,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "gather_valu_kernel (bf16, head_dim 128, 4 q heads per kv head, "
                               "token-index list)",
                     "kernel_avg_us": round(kern_avg * 1e3, 3),
                     "frac_of_stream_read": round(achieved / stream_ref["GBps"], 4),
                     "frac_of_address_replay": round(replay["us"] / (kern_avg * 1e3), 4),
                     "address_replay": replay,
                     "algorithmic_bytes_per_launch": a["algo_bytes"], "unit_of_work": a["unit"],
                     "units_per_launch": a["units"], "bytes_per_unit": a["per_unit"],
                     "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, scaled by a "
                                       "copy of known size; null when the sources changed since"},
    }
    del calls, ws, out
    torch.cuda.empty_cache()
    if not args.no_other_workloads:
        res["other_workloads"] = [run_other() for run_other in others.values()]
    if not args.no_cpu_baseline:
        log("cpu baseline (~%.0f s all threads + single-thread samples)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    bad = [] if par["ok"] else ["c2_decode_bf16"]
    bad += [w["workload"] for w in res.get("other_workloads", []) if not w["parity"]["ok"]]
    res["parity_ok"] = not bad
    print(json.dumps(res), flush=True)
    if bad:
        log("PARITY FAILED against the fp64 oracle: %s" % ", ".join(bad))
        sys.exit(3)


if __name__ == "__main__":
    main()
