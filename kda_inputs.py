"""Seeded synthetic inputs for the KDA mixer (shared by the oracle and the GPU side).

This module holds no step of the method: it only draws random tensors with the
shapes and distributions of the GLM-5.3 linear-attention layers and casts them
to the dtypes the GPU path receives.  Both the fp64 oracle and the HIP path are
fed the *same* cast values (bf16 values upcast to float64 are exact).

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream, float32 draws, in
this order): packed document lengths (packed workloads only), q, k, v, the
gate normal, the beta normal, the initial-state normal.
  * q, v ~ N(0, 1); k ~ N(0, 1) then L2-normalised over the head dim per
    (token, head), before the cast.
  * log_g = -softplus(N(0, 1)) * gate_scale   (a log-decay gate <= 0).
  * beta = sigmoid(N(0, 1)).
  * init_state ~ N(0, 0.02^2) per element, or zeros.
  * Packed document lengths floor(exp(U(ln lo, ln hi))) drawn until their sum
    reaches the total; the last one is truncated.
Layouts: q, k, log_g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
init_state [N, H, dk, dv]; cu_seqlens int32 [N+1].
Upstream gradients of the backward (their own stream, ``upstream_grads``):
d_out ~ N(0, 1) like out, d_final ~ N(0, 1) like the state.
Short convolution (``conv_inputs``, its own stream): x ~ N(0, 1), weight
~ N(0, 1/K), cache ~ N(0, 1).
"""
from __future__ import annotations

import math

import numpy as np
import torch

# The five workloads: shapes, dtypes, distributions and seeds.
CONFIGS = {
    # tiny oracle check: fp32 q/k/v, zero initial state, scale = 1/sqrt(16)
    "tiny": dict(kind="prefill", B=1, T=64, H=2, dk=16, dv=16, dtype="f32",
                 gate_scale=0.1, init="zeros", seed=0),
    # dense chunked prefill, 4 x 4096 tokens, 16 heads
    "prefill": dict(kind="prefill", B=4, T=4096, H=16, dk=128, dv=128, dtype="bf16",
                    gate_scale=0.05, init="normal", seed=1),
    # one packed row of 65536 tokens split into log-uniform documents, 32 heads
    "varlen": dict(kind="prefill", B=1, T=65536, H=32, dk=128, dv=128, dtype="bf16",
                   gate_scale=0.05, init="zeros", seed=2, doc_lo=64, doc_hi=16384),
    # decode: 256 sequences x 1 token
    "decode": dict(kind="step", B=256, T=1, H=32, dk=128, dv=128, dtype="bf16",
                   gate_scale=0.05, init="normal", seed=3),
    # batched verify: 64 sequences x 4 rows applied in order
    "verify": dict(kind="step", B=64, T=4, H=32, dk=128, dv=128, dtype="bf16",
                   gate_scale=0.05, init="normal", seed=4),
}


def doc_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> list[int]:
    """Log-uniform document lengths in [lo, hi] until ``total``; last one truncated."""
    lens, acc = [], 0
    while acc < total:
        n = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                seed: int = 0, gate_scale: float = 0.05, init: str = "normal",
                lengths=None, doc_lo: int | None = None, doc_hi: int | None = None,
                init_std: float = 0.02, gate_uniform: float | None = None) -> dict:
    """Draw one seeded workload.

    Dense when neither ``lengths`` nor ``doc_lo`` is given (B sequences of T
    tokens).  Packed when ``lengths`` (explicit document lengths summing to T)
    or ``doc_lo``/``doc_hi`` (drawn log-uniform) is given; then B must be 1.
    Returns CPU tensors: q, k, v (``dtype``), log_g, beta (float32),
    init_state (float32 or None), cu_seqlens (int32 or None), and ``scale``.
    ``gate_uniform`` = a replaces the gate recipe by log_g ~ U[-a, 0], taken
    from the same normal draws through the normal CDF (so every other tensor
    of the workload is unchanged).
    """
    rng = np.random.default_rng(seed)
    cu = None
    if doc_lo is not None:
        assert B == 1 and lengths is None
        lengths = doc_lengths(rng, T, doc_lo, doc_hi)
    if lengths is not None:
        assert B == 1 and sum(lengths) == T
        cu = cu_from_lengths(lengths)
    N = len(cu) - 1 if cu is not None else B

    q = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    k = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    k /= np.sqrt(np.sum(np.square(k, dtype=np.float64), axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    g = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    if gate_uniform is None:
        log_g = (-np.logaddexp(np.float32(0.0), g) * np.float32(gate_scale)).astype(np.float32)
    else:
        from scipy.special import ndtr
        log_g = (-float(gate_uniform) * ndtr(g.astype(np.float64))).astype(np.float32)
    del g
    b = rng.standard_normal((B, T, H), dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-b.astype(np.float64)))).astype(np.float32)
    s0 = None
    if init == "normal":
        s0 = rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(init_std)
    elif init != "zeros":
        raise ValueError(init)
    return dict(
        q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
        log_g=torch.from_numpy(log_g), beta=torch.from_numpy(beta),
        init_state=torch.from_numpy(s0) if s0 is not None else None,
        cu_seqlens=torch.from_numpy(cu.astype(np.int32)) if cu is not None else None,
        scale=dk ** -0.5, dtype=dtype, N=N,
    )


def upstream_grads(inp: dict, seed: int, final: bool = True, final_std: float = 1.0) -> dict:
    """Seeded upstream gradients for a workload drawn by ``make_inputs``:
    d_out ~ N(0, 1) shaped like out [B, T, H, dv] and, when ``final``,
    d_final ~ N(0, final_std^2) shaped like the state [N, H, dk, dv] (fp32)."""
    rng = np.random.default_rng(seed)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    d_out = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    d_final = None
    if final:
        d_final = rng.standard_normal((inp["N"], H, dk, dv), dtype=np.float32) * np.float32(final_std)
    return dict(d_out=torch.from_numpy(d_out), d_final=torch.from_numpy(d_final) if final else None)


def conv_inputs(B: int, T: int, channels: int, K: int, dtype: str = "bf16", seed: int = 0, lengths=None,
                cache: bool = True) -> dict:
    """Seeded inputs of the short convolution: x ~ N(0, 1) [B, T, channels]
    cast to ``dtype``; weight ~ N(0, 1/K) [channels, K] (fp32); init_cache ~
    N(0, 1) [N, channels, K-1] (fp32) when ``cache``; packed when ``lengths``
    (B == 1) is given."""
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        assert B == 1 and sum(lengths) == T
        cu = cu_from_lengths(lengths)
    N = len(cu) - 1 if cu is not None else B
    x = rng.standard_normal((B, T, channels), dtype=np.float32)
    w = rng.standard_normal((channels, K), dtype=np.float32) / np.float32(np.sqrt(K))
    c0 = rng.standard_normal((N, channels, K - 1), dtype=np.float32) if cache else None
    return dict(x=_cast(x, dtype), weight=torch.from_numpy(w),
                init_cache=torch.from_numpy(c0) if c0 is not None else None,
                cu_seqlens=torch.from_numpy(cu.astype(np.int32)) if cu is not None else None, N=N)


def config(name: str, **overrides) -> dict:
    """Inputs of one named workload (see ``CONFIGS``); keyword overrides allowed."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    c.pop("kind")
    return make_inputs(**c)


def to_f64(t: torch.Tensor | None):
    """Exact float64 numpy copy of a (bf16 / fp32) tensor, or None."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
