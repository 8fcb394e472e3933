"""Shared helpers of the GPU parity tests: error metric, device copies, the oracle."""
import os

import numpy as np
import torch

import oracle
from kda_inputs import to_f64

# Tolerances of the parity contract: max |gpu - oracle| / rms(oracle) over a
# whole output (or final-state) tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite GPU output"
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.abs(x - ref).max() / max(rms, 1e-30))


def to_dev(inp: dict, device="cuda"):
    out = {}
    for key in ("q", "k", "v", "log_g", "beta", "init_state", "cu_seqlens"):
        t = inp.get(key)
        out[key] = t.to(device).contiguous() if t is not None else None
    return out


def oracle_full(inp: dict):
    """Oracle on the whole problem.  Returns (out, final) float64."""
    cu = inp["cu_seqlens"].numpy().astype(np.int64) if inp["cu_seqlens"] is not None else None
    return oracle.kda_forward(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), to_f64(inp["log_g"]),
                              to_f64(inp["beta"]), init_state=to_f64(inp["init_state"]), cu_seqlens=cu,
                              scale=inp["scale"], n_threads=oracle_threads())
