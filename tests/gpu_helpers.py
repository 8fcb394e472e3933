"""Shared helpers of the GPU parity tests: error metric, oracle on chosen units."""
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


def oracle_units(inp: dict, units):
    """Oracle on sampled (sequence|document n, head h) units only.

    Returns {(n, h): (rows slice, out [len, dv], final [dk, dv])}, each unit run
    alone from its own initial state (documents never share state)."""
    q, k, v, g, b = inp["q"], inp["k"], inp["v"], inp["log_g"], inp["beta"]
    cu = inp["cu_seqlens"]
    res = {}
    for n, h in units:
        if cu is not None:
            a, e = int(cu[n]), int(cu[n + 1])
            bi, sl = 0, slice(a, e)
        else:
            bi, sl = n, slice(0, q.shape[1])
        pick = lambda t: to_f64(t[bi:bi + 1, sl, h:h + 1])
        s0 = inp["init_state"]
        s0 = to_f64(s0[n:n + 1, h:h + 1]) if s0 is not None else None
        out, fin = oracle.kda_forward(pick(q), pick(k), pick(v), pick(g), to_f64(b[bi:bi + 1, sl, h:h + 1]),
                                      init_state=s0, scale=inp["scale"], n_threads=1)
        res[(n, h)] = (bi, sl, out[0, :, 0], fin[0, 0])
    return res


def compare_units(ref: dict, out_gpu: torch.Tensor, fin_gpu: torch.Tensor, h_axis=2):
    """Concatenate the sampled units and return (err_out, err_final)."""
    og, orf, fg, frf = [], [], [], []
    out_c = out_gpu.detach().cpu()
    fin_c = fin_gpu.detach().cpu() if fin_gpu is not None else None
    for (n, h), (bi, sl, o, f) in ref.items():
        og.append(out_c[bi, sl, h].double().numpy())
        orf.append(o)
        if fin_c is not None:
            fg.append(fin_c[n, h].double().numpy())
            frf.append(f)
    e_out = err(np.concatenate(og), np.concatenate(orf))
    e_fin = err(np.stack(fg), np.stack(frf)) if fg else 0.0
    return e_out, e_fin
