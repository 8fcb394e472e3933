"""Python binding of libkda, the MI355X Kimi Delta Attention (KDA) mixer.

Thin ctypes layer over the C ABI declared in ``include/kda.h``: it checks
tensor shapes/dtypes/devices, allocates outputs with torch (device memory and
streams are torch's job), and passes raw device pointers plus torch's current
HIP stream.  Every step of the computation runs in the HIP kernels of
``libkda.so``; there is no CPU or PyTorch fallback.  The library is loaded on
first use, so the package (and its ``build`` module) imports before it is
built; any call then raises ``ImportError`` until ``libkda.so`` exists
(``python -m gated_delta_rule_67_amd.build``).

Outputs and workspaces this module allocates are allocated on the stream the
kernels run on (``stream``, else torch's current stream), so torch's caching
allocator never hands their memory to another stream while the kernels still
use it.

    out, final_state = chunk_fwd(q, k, v, log_g, beta, init_state=None, cu_seqlens=None)
    out = step(q, k, v, log_g, beta, state)        # state updated in place
    grads = chunk_bwd(q, k, v, log_g, beta, d_out, init_state=None, cu_seqlens=None, d_final=None)

Argument order follows ``_torch_recurrent_kda(q, k, v, g, beta, cu_seqlens)`` of
NeMo glm5_next.layers; q/k/v/g are [batch, seq, heads, head_dim], beta is
[batch, seq, heads].
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading

import torch

__all__ = ["chunk_fwd", "chunk_fwd_gated_norm", "chunk_fwd_static", "chunk_bwd", "step", "step_rows", "step_commit", "short_conv", "gated_rmsnorm",
           "workspace_bytes", "bwd_workspace_bytes", "abi_version", "KdaError", "LIB_PATH", "KDA_F32",
           "KDA_BF16", "KDA_FLAG_QK_L2NORM", "QK_L2NORM_EPS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
KDA_F32, KDA_BF16 = 0, 1
KDA_FLAG_QK_L2NORM = 1
STATIC_SCRATCH_BYTES = 64 << 20  # KDA_STATIC_SCRATCH_BYTES: the fixed scratch of chunk_fwd_static
QK_L2NORM_EPS = 1e-6  # eps inside the root of the in-kernel q / k L2 normalisation
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
           4: "KDA_ERR_ALIGN", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_UNSUPPORTED", 7: "KDA_ERR_HIP"}


class KdaDesc(ctypes.Structure):
    """Mirror of ``kda_desc`` in include/kda.h."""
    _fields_ = [("num_seqs", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libkda.so not found at {path}; build it with "
                          "`python -m gated_delta_rule_67_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, D = ctypes.c_void_p, ctypes.POINTER(KdaDesc)
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_chunk_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_workspace_bytes.argtypes = [D, ctypes.c_int]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.kda_chunk_fwd_gated_norm.restype = ctypes.c_int
    lib.kda_chunk_fwd_gated_norm.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P]
    lib.kda_chunk_fwd_static.restype = ctypes.c_int
    lib.kda_chunk_fwd_static.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [D, ctypes.c_int]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd.argtypes = [D] + [P] * 15 + [P]
    lib.kda_short_conv.restype = ctypes.c_int
    lib.kda_short_conv.argtypes = [D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P]
    lib.kda_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_gated_rmsnorm.argtypes = [D, P, P, P, ctypes.c_float, P, P]
    lib.kda_step.restype = ctypes.c_int
    lib.kda_step.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P, P]
    lib.kda_step_rows.restype = ctypes.c_int
    lib.kda_step_rows.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P, P, P]
    lib.kda_step_commit.restype = ctypes.c_int
    lib.kda_step_commit.argtypes = [D, P, P, P, P, P, ctypes.c_int32, P]
    return lib


_LIB = None
_LIB_LOCK = threading.Lock()


def _lib() -> ctypes.CDLL:
    """The loaded libkda.so (loaded once, on first use)."""
    global _LIB
    if _LIB is None:
        with _LIB_LOCK:
            if _LIB is None:
                _LIB = _load()
    return _LIB


def __getattr__(name):
    # ``gated_delta_rule_67_amd.lib``: the ctypes handle, loaded on first access
    if name == "lib":
        return _lib()
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def abi_version() -> int:
    return _lib().kda_abi_version()


def _check(status: int):
    if status != 0:
        raise KdaError(status, _lib().kda_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _need(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _allocates_on_launch_stream(fn):
    """Run ``fn`` with ``stream`` (when one is given) as torch's current
    stream, so the outputs and the workspace it allocates belong to the stream
    its kernels are enqueued on.  A workspace dropped on return then goes back
    to that stream's pool, where later allocations are ordered after the
    kernels that still use it."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return wrapper


def _out_code(dtype) -> int:
    if dtype == torch.float32:
        return KDA_F32
    if dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"out must be float32 or bfloat16, got {dtype}")


def make_desc(num_seqs, seq_len, H, dk, dv, qkv_dtype, scale=None, workspace=None, out_dtype=KDA_F32,
              flags=0) -> KdaDesc:
    d = KdaDesc()
    d.num_seqs, d.seq_len, d.num_heads, d.dk, d.dv = num_seqs, seq_len, H, dk, dv
    d.qkv_dtype, d.out_dtype, d.flags = qkv_dtype, out_dtype, flags
    d.scale = 0.0 if scale is None else float(scale)
    if workspace is not None:
        d.workspace, d.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return d


def workspace_bytes(num_seqs: int, seq_len: int, H: int, d: int, packed: bool,
                    qkv_dtype: int = KDA_BF16) -> int:
    """Device scratch bytes of a chunk_fwd call (see kda_chunk_workspace_bytes)."""
    desc = make_desc(num_seqs, seq_len, H, d, d, qkv_dtype)
    return _lib().kda_chunk_workspace_bytes(ctypes.byref(desc), int(packed))


@_allocates_on_launch_stream
def chunk_fwd(q, k, v, log_g, beta, init_state=None, cu_seqlens=None, scale=None,
              out=None, final_state=None, workspace=None, stream=None, out_dtype=torch.float32,
              qk_l2norm=False):
    """Chunked prefill.  Returns (out [B,T,H,dv], final_state [N,H,dk,dv] fp32).

    Dense: B sequences.  Packed: B == 1 and int32 ``cu_seqlens`` [N+1] on the
    device splits the row into N documents.  ``init_state`` [N,H,dk,dv] or None
    (zeros).  ``final_state`` may be passed (and may be ``init_state`` itself
    for an in-place resume); pass ``final_state=False`` to skip it.
    ``workspace`` (uint8 device tensor) is allocated when absent or too small.
    ``out_dtype`` float32 or bfloat16 (the dtype of ``out`` when passed);
    ``qk_l2norm`` L2-normalises every q and k row inside the kernels.
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(q, "q", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(log_g, "log_g", (B, T, H, dk), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed mode takes a single row (B == 1)")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        N, L = cu_seqlens.shape[0] - 1, T
    else:
        N, L = B, T
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (B, T, H, dv), out.dtype, dev)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    else:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    desc = make_desc(N, L, H, dk, dv, code, scale, out_dtype=_out_code(out.dtype),
                     flags=KDA_FLAG_QK_L2NORM if qk_l2norm else 0)
    need = _lib().kda_chunk_workspace_bytes(ctypes.byref(desc), int(cu_seqlens is not None))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        desc.workspace, desc.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(_lib().kda_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                             _ptr(init_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
                             _stream(stream)))
    return out, final_state


@_allocates_on_launch_stream
def chunk_fwd_gated_norm(q, k, v, log_g, beta, gate, norm_weight, eps, init_state=None, cu_seqlens=None, scale=None,
                         out=None, final_state=None, workspace=None, stream=None, out_dtype=torch.bfloat16,
                         qk_l2norm=False):
    """``chunk_fwd`` whose output passes the gated per-head RMSNorm in the same
    call: out = o / sqrt(mean(o^2) + eps) * norm_weight * sigmoid(gate) per
    (token, head), o written to ``out`` in its dtype and normalised there in
    place.  ``gate`` is shaped like the output with q's dtype, ``norm_weight``
    [dv] fp32.  Returns (out [B,T,H,dv] in ``out_dtype``, final_state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(log_g, "log_g", (B, T, H, dk), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(gate, "gate", (B, T, H, dv), dt, dev)
    _need(norm_weight, "norm_weight", (dv,), torch.float32, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed mode takes a single row (B == 1)")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        N, L = cu_seqlens.shape[0] - 1, T
    else:
        N, L = B, T
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (B, T, H, dv), out.dtype, dev)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    else:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    desc = make_desc(N, L, H, dk, dv, code, scale, out_dtype=_out_code(out.dtype),
                     flags=KDA_FLAG_QK_L2NORM if qk_l2norm else 0)
    need = _lib().kda_chunk_workspace_bytes(ctypes.byref(desc), int(cu_seqlens is not None))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        desc.workspace, desc.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(_lib().kda_chunk_fwd_gated_norm(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                                           _ptr(init_state), _ptr(cu_seqlens), _ptr(gate), _ptr(norm_weight),
                                           ctypes.c_float(eps), _ptr(out), _ptr(final_state), _stream(stream)))
    return out, final_state


def chunk_fwd_static(q, k, v, log_g, beta, out, final_state=None, init_state=None, cu_seqlens=None, scale=None,
                     stream=None, qk_l2norm=False):
    """``chunk_fwd`` through kda_chunk_fwd_static: the library's fixed scratch
    (STATIC_SCRATCH_BYTES per device) instead of a workspace, and no
    allocation here either: ``out`` [B,T,H,dv] (fp32 or bf16) and
    ``final_state`` [N,H,dk,dv] fp32 (or None) are the caller's.  Calls that
    overlap on one device share that scratch and must be ordered by the caller."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, name, shp in ((k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv))):
        _need(t, name, shp, dt, dev)
    _need(log_g, "log_g", (B, T, H, dk), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed mode takes a single row (B == 1)")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        N, L = cu_seqlens.shape[0] - 1, T
    else:
        N, L = B, T
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    _need(out, "out", (B, T, H, dv), out.dtype, dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    desc = make_desc(N, L, H, dk, dv, code, scale, out_dtype=_out_code(out.dtype),
                     flags=KDA_FLAG_QK_L2NORM if qk_l2norm else 0)
    _check(_lib().kda_chunk_fwd_static(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                                       _ptr(init_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
                                       _stream(stream)))
    return out, final_state


def bwd_workspace_bytes(num_seqs: int, seq_len: int, H: int, d: int, packed: bool) -> int:
    """Device scratch bytes of a chunk_bwd call (see kda_chunk_bwd_workspace_bytes)."""
    desc = make_desc(num_seqs, seq_len, H, d, d, KDA_BF16)
    return _lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(desc), int(packed))


@_allocates_on_launch_stream
def chunk_bwd(q, k, v, log_g, beta, d_out, init_state=None, cu_seqlens=None, d_final=None, scale=None,
              grads=None, d_init_state=True, workspace=None, stream=None):
    """Reverse mode of ``chunk_fwd``: gradients of sum(d_out * out) +
    sum(d_final * final_state) for the same inputs.

    Returns a dict of fp32 tensors ``dq, dk, dv, dlog_g, dbeta`` shaped like
    q, k, v, log_g, beta, and ``d_init_state`` [N, H, dk, dv] (None when
    ``d_init_state=False``).  ``grads`` may hold preallocated output tensors
    under the same keys.  ``workspace`` (uint8 device tensor) is allocated when
    absent or too small.
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(log_g, "log_g", (B, T, H, dk), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(d_out, "d_out", (B, T, H, dv), torch.float32, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed mode takes a single row (B == 1)")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        N, L = cu_seqlens.shape[0] - 1, T
    else:
        N, L = B, T
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    if d_final is not None:
        _need(d_final, "d_final", (N, H, dk, dv), torch.float32, dev)
    shapes = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv), "dlog_g": (B, T, H, dk),
              "dbeta": (B, T, H), "d_init_state": (N, H, dk, dv)}
    g = dict(grads or {})
    for name, shp in shapes.items():
        if name == "d_init_state" and d_init_state is False:
            g[name] = None
            continue
        if g.get(name) is None:
            g[name] = torch.empty(shp, dtype=torch.float32, device=dev)
        else:
            _need(g[name], name, shp, torch.float32, dev)
    desc = make_desc(N, L, H, dk, dv, code, scale)
    need = _lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(desc), int(cu_seqlens is not None))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        desc.workspace, desc.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(_lib().kda_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                             _ptr(init_state), _ptr(cu_seqlens), _ptr(d_out), _ptr(d_final), _ptr(g["dq"]),
                             _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_g"]), _ptr(g["dbeta"]),
                             _ptr(g["d_init_state"]), _stream(stream)))
    return g


@_allocates_on_launch_stream
def short_conv(x, weight, cu_seqlens=None, init_cache=None, activation=0, out=None, final_cache=None,
               stream=None):
    """Short causal depthwise convolution of x [B, T, channels] (fp32 or bf16)
    with ``weight`` [channels, K] (fp32), resetting at the documents of
    ``cu_seqlens`` (packed, B == 1).  ``init_cache`` [N, channels, K-1] holds
    the K-1 inputs before each sequence (None: zeros).  ``activation`` 0 is the
    identity, 1 SiLU.  Returns (out like x, final_cache [N, channels, K-1]
    fp32); pass ``final_cache=False`` to skip it, or a tensor (it may be
    ``init_cache`` itself for dense sequences of 1, 2, 4, 8, 16 or 32 tokens)."""
    B, T, Cn = x.shape
    K = weight.shape[1]
    dev = x.device
    code = _dtype_code(x)
    _need(weight, "weight", (Cn, K), torch.float32, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed mode takes a single row (B == 1)")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        N, L = cu_seqlens.shape[0] - 1, T
    else:
        N, L = B, T
    if init_cache is not None:
        _need(init_cache, "init_cache", (N, Cn, K - 1), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", (B, T, Cn), x.dtype, dev)
    if final_cache is None:
        final_cache = torch.empty((N, Cn, K - 1), dtype=torch.float32, device=dev)
    elif final_cache is False:
        final_cache = None
    else:
        _need(final_cache, "final_cache", (N, Cn, K - 1), torch.float32, dev)
    desc = make_desc(N, L, 1, 16, 16, code)
    fc = final_cache if (final_cache is not None and final_cache.numel() > 0) else None
    ic = init_cache if (init_cache is not None and init_cache.numel() > 0) else None
    _check(_lib().kda_short_conv(ctypes.byref(desc), Cn, K, int(activation), _ptr(x), _ptr(weight), _ptr(cu_seqlens),
                              _ptr(ic), _ptr(out), _ptr(fc), _stream(stream)))
    return out, final_cache


@_allocates_on_launch_stream
def gated_rmsnorm(o, gate, weight, eps, out=None, out_dtype=torch.bfloat16, stream=None):
    """Gated per-head RMSNorm of the mixer output o [B, T, H, D] (fp32) with
    ``gate`` like o (fp32 or bf16) and ``weight`` [D] (fp32):
    o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate) per (token, head).
    Returns out [B, T, H, D] in ``out_dtype`` (bf16 or fp32; ``out`` may be o
    itself when fp32)."""
    B, T, H, D = o.shape
    dev = o.device
    _need(o, "o", (B, T, H, D), torch.float32, dev)
    _need(gate, "gate", (B, T, H, D), gate.dtype, dev)
    g_code = _dtype_code(gate)
    _need(weight, "weight", (D,), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, D), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (B, T, H, D), out.dtype, dev)
    desc = make_desc(B, T, H, D, D, g_code)
    desc.out_dtype = _dtype_code(out)
    _check(_lib().kda_gated_rmsnorm(ctypes.byref(desc), _ptr(o), _ptr(gate), _ptr(weight), ctypes.c_float(eps),
                                 _ptr(out), _stream(stream)))
    return out


@_allocates_on_launch_stream
def step(q, k, v, log_g, beta, state, scale=None, out=None, stream=None, out_dtype=torch.float32,
         qk_l2norm=False):
    """Decode (n_tok = 1) or multi-row verify: rows [N, n_tok, H, d] applied in
    order to ``state`` [N, H, dk, dv] (fp32), which is updated in place.
    Returns out [N, n_tok, H, dv] (``out_dtype``: float32 or bfloat16)."""
    N, n_tok, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(k, "k", (N, n_tok, H, dk), dt, dev)
    _need(v, "v", (N, n_tok, H, dv), dt, dev)
    _need(log_g, "log_g", (N, n_tok, H, dk), torch.float32, dev)
    _need(beta, "beta", (N, n_tok, H), torch.float32, dev)
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, n_tok, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (N, n_tok, H, dv), out.dtype, dev)
    desc = make_desc(N, n_tok, H, dk, dv, code, scale, out_dtype=_out_code(out.dtype),
                     flags=KDA_FLAG_QK_L2NORM if qk_l2norm else 0)
    _check(_lib().kda_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                        _ptr(state), ctypes.c_int32(n_tok), _ptr(out), _stream(stream)))
    return out


@_allocates_on_launch_stream
def step_rows(q, k, v, log_g, beta, state, scale=None, out=None, deltas=None, stream=None,
              out_dtype=torch.float32, qk_l2norm=False):
    """Speculative verify, first half: the outputs of rows [N, n_tok, H, d] as
    ``step`` would give them, with ``state`` left unchanged.  Returns (out,
    deltas), both [N, n_tok, H, dv] (out in ``out_dtype``, deltas fp32);
    ``deltas`` feeds ``step_commit``."""
    N, n_tok, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(k, "k", (N, n_tok, H, dk), dt, dev)
    _need(v, "v", (N, n_tok, H, dv), dt, dev)
    _need(log_g, "log_g", (N, n_tok, H, dk), torch.float32, dev)
    _need(beta, "beta", (N, n_tok, H), torch.float32, dev)
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, n_tok, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (N, n_tok, H, dv), out.dtype, dev)
    if deltas is None:
        deltas = torch.empty((N, n_tok, H, dv), dtype=torch.float32, device=dev)
    else:
        _need(deltas, "deltas", (N, n_tok, H, dv), torch.float32, dev)
    desc = make_desc(N, n_tok, H, dk, dv, code, scale, out_dtype=_out_code(out.dtype),
                     flags=KDA_FLAG_QK_L2NORM if qk_l2norm else 0)
    _check(_lib().kda_step_rows(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta),
                             _ptr(state), ctypes.c_int32(n_tok), _ptr(out), _ptr(deltas), _stream(stream)))
    return out, deltas


def step_commit(k, log_g, deltas, state, accept, stream=None, qk_l2norm=False):
    """Speculative verify, second half: advance each sequence n of ``state``
    (in place) by its first ``accept[n]`` rows (int32 [N] on the device), from
    the ``deltas`` that ``step_rows`` returned for the same rows and state
    (``qk_l2norm`` as given to ``step_rows``)."""
    N, n_tok, H, dk = k.shape
    dv = deltas.shape[-1]
    dev = k.device
    code = _dtype_code(k)
    _need(log_g, "log_g", (N, n_tok, H, dk), torch.float32, dev)
    _need(deltas, "deltas", (N, n_tok, H, dv), torch.float32, dev)
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    _need(accept, "accept", (N,), torch.int32, dev)
    desc = make_desc(N, n_tok, H, dk, dv, code, None, flags=KDA_FLAG_QK_L2NORM if qk_l2norm else 0)
    _check(_lib().kda_step_commit(ctypes.byref(desc), _ptr(k), _ptr(log_g), _ptr(deltas), _ptr(accept),
                               _ptr(state), ctypes.c_int32(n_tok), _stream(stream)))
