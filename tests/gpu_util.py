"""Helpers for the GPU parity tests: compare the HIP path with the fp64 oracle."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

# Max-abs tolerances on outputs of unit-variance inputs, per element type.
TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}
# Default relative-RMS gates (||got - ref||_2 / ||ref||_2), per element type. Outputs
# of attention over many keys are small (std 0.02-0.08 at the workloads' shapes), so
# the max-abs bound alone would pass a result that lost a key block; the relative gate
# does not. fp32: fp32 accumulation only (measured 1e-7 to 3e-7). bf16: the weights P
# enter P.V rounded to bf16 and bf16 outputs are rounded to nearest even, each with
# relative error below 2^-8 (measured 1e-3 to 2.4e-3 over the suite). e4m3: inputs
# decode exactly, so the arithmetic error is the bf16 case's (measured 2.3e-3).
REL = {"f32": 2e-6, "bf16": 1e-2, "e4m3": 1e-2}

_LOG = os.environ.get("QSA_PARITY_LOG")


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def compare(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str, rel_rms_max: float = None):
    """Element-by-element check: finite, max |got - ref| <= TOL[dtype] and relative RMS
    error <= rel_rms_max (default REL[dtype]). Returns (max_abs, rel_rms)."""
    g = to64(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.isfinite(g).all(), "%s: non-finite output (%d values)" % (what, (~np.isfinite(g)).sum())
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    rel = float(np.sqrt((err ** 2).mean()) / denom) if denom > 0 else float(np.sqrt((err ** 2).mean()) if err.size else 0.0)
    gate = REL[dtype] if rel_rms_max is None else rel_rms_max
    if _LOG:
        with open(_LOG, "a") as f:
            f.write(json.dumps({"what": what, "dtype": dtype, "max_abs": max_abs, "tol": TOL[dtype],
                                "rel_rms": rel, "rel_gate": gate, "ref_rms": denom}) + "\n")
    assert max_abs <= TOL[dtype], "%s: max abs err %.3e > %.1e (rel-RMS %.2e)" % (what, max_abs, TOL[dtype], rel)
    assert rel <= gate, "%s: rel-RMS %.3e > %.1e (max abs %.2e)" % (what, rel, gate, max_abs)
    return max_abs, rel


def log_value(what: str, **values):
    """Record a measured figure in the parity log (when QSA_PARITY_LOG names one)."""
    if _LOG:
        with open(_LOG, "a") as f:
            f.write(json.dumps(dict(what=what, **values)) + "\n")


def announce(msg: str):
    print("[gpu-test] " + msg, flush=True)
