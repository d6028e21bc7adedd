"""Helpers for the GPU parity tests: compare the HIP path with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

# Max-abs tolerances on outputs of unit-variance inputs, per element type.
TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def compare(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str, rel_rms_max: float = None):
    """Element-by-element check: finite, max |got - ref| <= TOL[dtype]; optional rel-RMS gate.
    Returns (max_abs, rel_rms)."""
    g = to64(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.isfinite(g).all(), "%s: non-finite output (%d values)" % (what, (~np.isfinite(g)).sum())
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    rel = float(np.sqrt((err ** 2).mean()) / denom) if denom > 0 else 0.0
    assert max_abs <= TOL[dtype], "%s: max abs err %.3e > %.1e (rel-RMS %.2e)" % (what, max_abs, TOL[dtype], rel)
    if rel_rms_max is not None:
        assert rel <= rel_rms_max, "%s: rel-RMS %.3e > %.1e" % (what, rel, rel_rms_max)
    return max_abs, rel


def announce(msg: str):
    print("[gpu-test] " + msg, flush=True)
