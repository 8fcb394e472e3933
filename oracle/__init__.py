"""fp64 CPU oracle of the Kimi Delta Attention recurrence (Python loader).

TEST INFRASTRUCTURE ONLY.  The correctness reference for the GPU path.  Only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``libkda`` and the
``gated_delta_rule_67_amd`` binding) never imports it, and it imports nothing
from the product path.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, libm ``exp``): the
token loop of the gated delta rule as printed in the GLM-5.3-Flash model notes
(Glm5NextTextLinearAttention snippet), with the output read from the updated
state, and packed documents reset at their boundaries (NeMo glm5_next.layers,
``_torch_recurrent_kda``), optionally on L2-normalised query and key rows
(``qk_l2norm``); its reverse mode, the same loop differentiated
token by token (that page documents the recurrence as differentiable); and the
short causal depthwise convolution that feeds q, k and v
(``_TorchShortConvolution``); and the gated per-head RMSNorm on the output
(``_TorchRMSNormGated``).  This module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")

_lib = None


def build(out_path: str = LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", *extra_flags, src, "-o", out_path, "-lm"]
    tmp = out_path + ".tmp"
    cmd[cmd.index(out_path)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def load(path: str = LIB_PATH):
    """Load a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
    lib.kda_oracle_forward.restype = ctypes.c_int
    lib.kda_oracle_forward.argtypes = [i64, i64, i64, i64, i64, dp, dp, dp, dp, dp,
                                       dp, ip, ctypes.c_double, dp, dp, ctypes.c_int]
    lib.kda_oracle_backward.restype = ctypes.c_int
    lib.kda_oracle_backward.argtypes = [i64, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp, ip,
                                        ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.kda_oracle_short_conv.restype = ctypes.c_int
    lib.kda_oracle_short_conv.argtypes = [i64, i64, i64, i64, dp, dp, ip, dp, ctypes.c_int, dp, dp, ctypes.c_int]
    lib.kda_oracle_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_oracle_gated_rmsnorm.argtypes = [i64, i64, dp, dp, dp, ctypes.c_double, dp]
    lib.kda_oracle_qk_l2norm.restype = ctypes.c_int
    lib.kda_oracle_qk_l2norm.argtypes = [i64, i64, ctypes.c_double, dp, dp, dp, dp]
    lib.kda_oracle_threads.restype = ctypes.c_int
    lib.kda_oracle_threads.argtypes = [ctypes.c_int]
    return lib


def _get_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load()
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def threads(n_threads: int = 0) -> int:
    return _get_lib().kda_oracle_threads(n_threads)


QK_L2_EPS = 1e-6  # eps inside the root of the optional q / k L2 normalisation


def qk_l2norm(q, k, eps: float = QK_L2_EPS, lib=None):
    """Each (token, head) row of q and of k divided by sqrt(sum of squares +
    eps).  q, k: [..., D].  Returns (qn, kn) in float64."""
    lib = lib or _get_lib()
    q, k = _f64(q), _f64(k)
    assert q.shape == k.shape
    D = q.shape[-1]
    qn, kn = np.zeros(q.shape), np.zeros(k.shape)
    rc = lib.kda_oracle_qk_l2norm(q.size // D, D, float(eps), _ptr(q), _ptr(k), _ptr(qn), _ptr(kn))
    if rc != 0:
        raise ValueError(f"kda_oracle_qk_l2norm failed with code {rc}")
    return qn, kn


def kda_forward(q, k, v, log_g, beta, init_state=None, cu_seqlens=None,
                scale=None, n_threads: int = 0, lib=None, qk_l2norm_eps=None):
    """Run the token-loop recurrence.

    q, k, log_g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H].
    Dense: B independent sequences.  Packed: B == 1 and ``cu_seqlens`` [N+1]
    splits the row into N documents, each starting from its own initial state.
    init_state: [N, H, dk, dv] or None (zeros).  scale defaults to dk**-0.5.
    ``qk_l2norm_eps`` (a float) first L2-normalises every row of q and k
    (:func:`qk_l2norm`); None leaves them as given.
    Returns (out [B, T, H, dv], final_state [N, H, dk, dv]) in float64.
    """
    lib = lib or _get_lib()
    q, k, v, log_g, beta = (_f64(x) for x in (q, k, v, log_g, beta))
    if qk_l2norm_eps is not None:
        q, k = qk_l2norm(q, k, qk_l2norm_eps, lib=lib)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and log_g.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if cu_seqlens is not None:
        assert B == 1, "packed mode takes one row"
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N, L = cu.shape[0] - 1, T
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        cu, N, L, cu_p = None, B, T, None
    if scale is None:
        scale = dk ** -0.5
    s0 = _f64(init_state) if init_state is not None else None
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    out = np.zeros((B, T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = lib.kda_oracle_forward(N, L, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(log_g),
                                _ptr(beta), _ptr(s0), cu_p, float(scale), _ptr(out),
                                _ptr(fin), int(n_threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_forward failed with code {rc}")
    return out, fin


def kda_step(q, k, v, log_g, beta, state, scale=None, n_threads: int = 0, qk_l2norm_eps=None):
    """Decode / verify: n_tok rows per sequence applied in order from ``state``.

    Rows are [N, n_tok, H, d]; row t of a sequence is applied after rows < t
    (metrale glm5next_layer invariants: verify row t uses slot t).  Returns
    (out [N, n_tok, H, dv], new_state [N, H, dk, dv]); ``state`` is not modified.
    """
    return kda_forward(q, k, v, log_g, beta, init_state=state, scale=scale,
                       n_threads=n_threads, qk_l2norm_eps=qk_l2norm_eps)


def kda_backward(q, k, v, log_g, beta, init_state=None, cu_seqlens=None, scale=None,
                 d_out=None, d_final=None, n_threads: int = 0, lib=None):
    """Gradients of L = sum(d_out * out) + sum(d_final * final_state).

    Inputs as for :func:`kda_forward`; ``d_out`` [B, T, H, dv] and ``d_final``
    [N, H, dk, dv] may be None (zeros).  Returns a dict of float64 arrays
    ``dq, dk, dv, dlog_g, dbeta, d_init_state`` shaped like q, k, v, log_g,
    beta and the initial state.
    """
    lib = lib or _get_lib()
    q, k, v, log_g, beta = (_f64(x) for x in (q, k, v, log_g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and log_g.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if cu_seqlens is not None:
        assert B == 1, "packed mode takes one row"
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N, L = cu.shape[0] - 1, T
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        cu, N, L, cu_p = None, B, T, None
    if scale is None:
        scale = dk ** -0.5
    s0 = _f64(init_state) if init_state is not None else None
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    do = _f64(d_out) if d_out is not None else None
    if do is not None:
        assert do.shape == (B, T, H, dv)
    dfin = _f64(d_final) if d_final is not None else None
    if dfin is not None:
        assert dfin.shape == (N, H, dk, dv)
    g = {"dq": np.zeros(q.shape), "dk": np.zeros(q.shape), "dv": np.zeros(v.shape),
         "dlog_g": np.zeros(q.shape), "dbeta": np.zeros(beta.shape), "d_init_state": np.zeros((N, H, dk, dv))}
    rc = lib.kda_oracle_backward(N, L, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                                 _ptr(s0), cu_p, float(scale), _ptr(do), _ptr(dfin), _ptr(g["dq"]),
                                 _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_g"]), _ptr(g["dbeta"]),
                                 _ptr(g["d_init_state"]), int(n_threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_backward failed with code {rc}")
    return g


def short_conv(x, w, cu_seqlens=None, init_cache=None, act: int = 0, n_threads: int = 0, lib=None):
    """Short causal depthwise convolution.

    x: [B, T, channels] (dense: B sequences; packed: B == 1 with ``cu_seqlens``
    [N+1]); w: [channels, K]; init_cache: [N, channels, K-1] or None (zeros);
    act 0 = identity, 1 = SiLU.  Returns (y [B, T, channels],
    final_cache [N, channels, K-1]) in float64.
    """
    lib = lib or _get_lib()
    x, w = _f64(x), _f64(w)
    B, T, Cn = x.shape
    K = w.shape[1]
    assert w.shape == (Cn, K)
    if cu_seqlens is not None:
        assert B == 1, "packed mode takes one row"
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N, L = cu.shape[0] - 1, T
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        cu, N, L, cu_p = None, B, T, None
    c0 = _f64(init_cache) if init_cache is not None else None
    if c0 is not None:
        assert c0.shape == (N, Cn, K - 1)
    y = np.zeros((B, T, Cn))
    fin = np.zeros((N, Cn, K - 1))
    rc = lib.kda_oracle_short_conv(N, L, Cn, K, _ptr(x), _ptr(w), cu_p, _ptr(c0), int(act), _ptr(y), _ptr(fin),
                                   int(n_threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_short_conv failed with code {rc}")
    return y, fin


def gated_rmsnorm(o, g, w, eps: float, lib=None):
    """Gated per-head RMSNorm over the last axis: o, g [..., D]; w [D].
    Returns y shaped like o (float64)."""
    lib = lib or _get_lib()
    o, g, w = _f64(o), _f64(g), _f64(w)
    assert g.shape == o.shape and w.shape == (o.shape[-1],)
    D = o.shape[-1]
    rows = o.size // D
    y = np.zeros(o.shape)
    rc = lib.kda_oracle_gated_rmsnorm(rows, D, _ptr(o), _ptr(g), _ptr(w), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError(f"kda_oracle_gated_rmsnorm failed with code {rc}")
    return y
