"""Benchmark of libkda on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --only {prefill,varlen,step,backward,conv,norm,copy}      (profiling runs)
    python bench.py [--traffic-kind {prefill,backward}] --traffic-from FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR

A step is one kda_chunk_fwd call (chunked prefill) over the dense workload
B=4 x T=4096 tokens, H=16 heads, dk=dv=128, bf16 q/k/v, fp32 gates/beta/state,
fp32 out, with inputs resident in HBM.  ``value`` is prefill tokens/s
(tokens of the 16-head mixer per second).  The same JSON line carries:
  roofline      prefill kernel: algorithmic bytes per launch / mean launch time
                (HIP events on the launch stream) against 8 TB/s HBM
  mfma          algorithmic prefill FLOP/s against the 2516.6 TFLOP/s dense
                16-bit MFMA peak
  varlen        the packed 65536-token, 32-head prefill: tokens/s and its own
                HBM roofline (beside the headline, not part of it)
  gated_rmsnorm kda_gated_rmsnorm on the dense workload's output (fp32 o,
                bf16 gate and out): its own HBM roofline
  short_conv    kda_short_conv over q, k, v of the dense workload (6144
                channels, width 4, bf16): its own HBM roofline
  backward      kda_chunk_bwd on the dense workload: tokens/s and its roofline
                against the 157.3 TFLOP/s fp32 peak (it computes in fp32)
  verify_rollback  the 64 x 4-row verify split into kda_step_rows (state read
                only) and kda_step_commit, each with its own HBM roofline
  decode/verify kda_step GB/s on 256 x 1 and 64 x 4 rows, H=32, d=128, each
                with its own roofline (state read + write + row traffic)
  cpu_baseline  the fp64 oracle timed on the host on a bounded sample of the
                same prefill workload
Every timed region follows SETTLE_S seconds of the same workload run back to
back (untimed), then the W warm-up steps: the GPU's clocks need some 30 ms
of sustained load to reach their steady state.
Only one GPU is used; --gpus above 1 exits with a message.

roofline.traffic is the HBM bytes of one prefill call measured with rocprofv3
counters (FETCH_SIZE, WRITE_SIZE; one pass each), scaled by what the same
counters read for a plain copy of known size (--only copy).  --traffic-from
turns those four runs' CSV output into profiles/traffic_prefill_dense.txt
(--traffic-kind backward: profiles/traffic_backward_dense.txt, for the
backward's roofline), stamped with a hash of the kernel sources; the figure is
reported only while the sources still hash the same (else null).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kda_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2516.6      # MI355X dense fp16/bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (matrix and vector), TFLOP/s
CHUNK = 64
COPY_BYTES = 512 << 20         # calibration copy: bytes read (= bytes written)
# Counter-measured HBM traffic per call, one summary per measured path: the
# file, the sources that define its kernels (their code, not the ABI around
# them), the kernels summed, and the workload the counters were taken on.
TRAFFIC = {
    "prefill": dict(file=os.path.join(ROOT, "profiles", "traffic_prefill_dense.txt"),
                    sources=["kda_twopass.hip", "kda_common.h", "kda_fallback.h"],
                    kernels=("prep_kernel", "scan_kernel"),
                    what="one kda_chunk_fwd call, dense 4 x 4096 tokens, 16 heads, d = 128, bf16"),
    "backward": dict(file=os.path.join(ROOT, "profiles", "traffic_backward_dense.txt"),
                     sources=["kda_backward.hip", "kda_common.h"],
                     kernels=("bwd_prep", "bwd_fscan", "bwd_rscan", "bwd_gstate", "bwd_gpairs"),
                     what="one kda_chunk_bwd call, dense 4 x 4096 tokens, 16 heads, d = 128, bf16"),
}
TRAFFIC_FILE = TRAFFIC["prefill"]["file"]
KERNEL_SOURCES = TRAFFIC["prefill"]["sources"]


def sources_hash(kind: str = "prefill") -> str:
    h = hashlib.sha256()
    for f in TRAFFIC[kind]["sources"]:
        with open(os.path.join(ROOT, "gated_delta_rule_67_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kind: str = "prefill"):
    """HBM bytes per call from the committed counter summary, or None when it
    is missing or was taken on other kernel sources."""
    try:
        kv = {}
        for line in open(TRAFFIC[kind]["file"]):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("sources_sha256") != sources_hash(kind):
            return None
        return int(kv["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def _counter_sums(run_dir: str, counter: str):
    """{kernel name: mean per-dispatch value} of one rocprofv3 --pmc csv run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in out.items()}


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kind="prefill"):
    fe, wr = _counter_sums(fetch_dir, "FETCH_SIZE"), _counter_sums(write_dir, "WRITE_SIZE")
    cf, cw = _counter_sums(copy_fetch_dir, "FETCH_SIZE"), _counter_sums(copy_write_dir, "WRITE_SIZE")
    pick = lambda d, pat: sum(v for k, v in d.items() if pat in k)
    copy_f = max(cf.values())   # the copy is the largest dispatch of its run
    copy_w = max(cw.values())
    k_fetch = COPY_BYTES / (copy_f * 1024.0)
    k_write = COPY_BYTES / (copy_w * 1024.0)
    lines = [f"sources_sha256: {sources_hash(kind)}",
             f"copy_fetch_kib: {copy_f:.1f}", f"copy_write_kib: {copy_w:.1f}",
             f"fetch_scale: {k_fetch:.4f}", f"write_scale: {k_write:.4f}"]
    total = 0.0
    for pat in TRAFFIC[kind]["kernels"]:
        f, w = pick(fe, pat), pick(wr, pat)
        b = f * 1024 * k_fetch + w * 1024 * k_write
        total += b
        lines += [f"{pat}_fetch_kib: {f:.1f}", f"{pat}_write_kib: {w:.1f}", f"{pat}_bytes: {b:.0f}"]
    lines.append(f"traffic_bytes_per_call: {total:.0f}")
    return lines


def prefill_bytes(tokens: int, H: int, d: int, n_states: int, qkv_bytes=2) -> int:
    """Algorithmic HBM bytes of one prefill call: q, k, v, log_g, beta in;
    out (fp32) out; initial and final states once per unit."""
    per_token_head = 3 * d * qkv_bytes + d * 4 + 4 + d * 4
    return tokens * H * per_token_head + 2 * n_states * H * d * d * 4


def prefill_flops(tokens: int, H: int, d: int) -> int:
    """Algorithmic FLOP of the chunked form per token-head: five C x d and three
    d x d products per token (dense tiles), 5*2*C*d + 3*2*d*d."""
    return tokens * H * (5 * 2 * CHUNK * d + 3 * 2 * d * d)


def step_bytes(N: int, n_tok: int, H: int, d: int, qkv_bytes=2) -> int:
    per_token_head = 3 * d * qkv_bytes + d * 4 + 4 + d * 4
    return N * H * 2 * d * d * 4 + N * n_tok * H * per_token_head


def backward_bytes(tokens: int, H: int, d: int, n_states: int, qkv_bytes=2) -> int:
    """Algorithmic HBM bytes of one kda_chunk_bwd call: q, k, v, log_g, beta
    and d_out in; dq, dk, dv, dlog_g (fp32) and dbeta out; per unit the
    initial state and d_final in, d_init_state out."""
    per_token_head = 3 * d * qkv_bytes + d * 4 + 4 + d * 4 + 4 * d * 4 + 4
    return tokens * H * per_token_head + 3 * n_states * H * d * d * 4


def backward_flops(tokens: int, H: int, d: int) -> int:
    """Algorithmic FLOP of the chunk-form reverse mode per token-head, 2 x the
    multiply-adds per 64-token chunk divided by 64: C^3/6 (the triangular
    inverse) + 6 C^2 d (pair matrices, W and U, the triangular products of the
    two scans and of the gradients) + 8 C d^2 (the C x d x d products: two in
    the forward scan, three in the reverse scan, three in the gradients)."""
    C = CHUNK
    macs_per_chunk = C ** 3 // 6 + 6 * C * C * d + 8 * C * d * d
    return tokens * H * 2 * macs_per_chunk // C


SETTLE_S = 0.2  # untimed sustained load before the warm-up steps


def settle(fn, seconds: float = SETTLE_S):
    """Run fn back to back for about ``seconds`` (untimed).  Under sustained
    load the GPU's clocks take some 30 ms to reach their steady state (the
    dense prefill runs at about 310 us per call for its first 20 calls and
    270 us from the 100th on; one idle second undoes it), so every timed
    region starts from that steady state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def timed_calls(fn, steps: int, warmup: int):
    """Settle, run fn warmup times, then steps times bracketed by
    synchronisation.  Returns (wall seconds of the timed region, per-call
    event milliseconds).  One pair of HIP events on the launch stream spans
    the steps calls and the mean call is their time over steps: an event
    recorded between two calls holds the next call's first kernel back until
    the event has been signalled, a gap the calls themselves do not have."""
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) / steps] * steps


def to_dev(inp):
    return {k: (inp[k].cuda().contiguous() if inp[k] is not None else None)
            for k in ("q", "k", "v", "log_g", "beta", "init_state", "cu_seqlens")}


def bench_prefill(kda, steps, warmup):
    inp = kda_inputs.config("prefill")
    d = to_dev(inp)
    B, T, H, D = inp["q"].shape
    out = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    fin = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")

    def call():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"],
                      out=out, final_state=fin)

    wall, ms = timed_calls(call, steps, warmup)
    tokens = B * T
    return dict(inp=inp, wall=wall, ms=ms, tokens=tokens, H=H, D=D,
                bytes=prefill_bytes(tokens, H, D, n_states=B), flops=prefill_flops(tokens, H, D))


def bench_varlen(kda, steps, warmup):
    """The packed workload: 65536 tokens split into documents of log-uniform
    length, H=32, d=128, bf16, zero initial states; timed like the dense
    prefill (back-to-back calls, HIP events around them).  Reported beside the
    headline, not as it."""
    inp = kda_inputs.config("varlen")
    d = to_dev(inp)
    B, T, H, D = inp["q"].shape
    N = d["cu_seqlens"].numel() - 1
    out = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")

    def call():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                      out=out, final_state=fin)

    wall, ms = timed_calls(call, steps, warmup)
    avg = float(np.mean(ms))
    nbytes = prefill_bytes(T, H, D, n_states=0) + N * H * D * D * 4  # final states only (zero initial)
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"workload": f"packed varlen prefill, 1 x {T} tokens in {N} documents (log-uniform 64..16384), "
                        f"H={H}, dk=dv={D}, bf16 q/k/v, zero initial states",
            "tokens_per_s": round(T / (wall / steps), 1), "us_per_call": round(avg * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "algorithmic_bytes": nbytes}


def bench_backward(kda, steps, warmup):
    """kda_chunk_bwd on the dense prefill workload (4 x 4096 tokens, H = 16,
    d = 128, bf16 q/k/v) with seeded upstream gradients, timed like the
    prefill (back-to-back calls, HIP events around them).  The backward computes
    in fp32 on the matrix cores, so its roofline is the fp32 peak."""
    inp = kda_inputs.config("prefill")
    up = kda_inputs.upstream_grads(inp, seed=240)
    d = to_dev(inp)
    B, T, H, D = inp["q"].shape
    do, dfin = up["d_out"].cuda(), up["d_final"].cuda()
    ws = torch.empty(kda.bwd_workspace_bytes(B, T, H, D, False), dtype=torch.uint8, device="cuda")
    grads = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], do, init_state=d["init_state"],
                          d_final=dfin, workspace=ws)

    def call():
        kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], do, init_state=d["init_state"], d_final=dfin,
                      grads=grads, workspace=ws)

    wall, ms = timed_calls(call, steps, warmup)
    avg = float(np.mean(ms))
    tokens = B * T
    fl, nb = backward_flops(tokens, H, D), backward_bytes(tokens, H, D, n_states=B)
    tf = fl / (avg * 1e-3) / 1e12
    return {"workload": f"dense backward, {B} x {T} tokens, H={H}, dk=dv={D}, bf16 q/k/v, fp32 gradients, "
                        "seeded d_out and d_final",
            "tokens_per_s": round(tokens / (wall / steps), 1), "us_per_call": round(avg * 1e3, 2),
            "algorithmic_flops": fl, "algorithmic_bytes": nb,
            "hbm_gbs": round(nb / (avg * 1e-3) / 1e9, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP32_PEAK_TFLOPS, 4), "traffic": read_traffic("backward")},
            "workspace_bytes": int(ws.numel())}


def conv_bytes(tokens: int, channels: int, K: int, n_seqs: int, x_bytes=2) -> int:
    """Algorithmic HBM bytes of one kda_short_conv call: x read and out
    written once, the fp32 weights, the final cache written (zero initial
    cache)."""
    return tokens * channels * 2 * x_bytes + channels * K * 4 + n_seqs * channels * (K - 1) * 4


def bench_conv(kda, steps, warmup):
    """kda_short_conv over q, k and v of the dense workload side by side
    (4 x 4096 tokens, 3 x 16 heads x 128 = 6144 channels, bf16), width 4,
    identity activation, zero caches, final cache written; timed like the
    prefill."""
    B, T, Cn, K = 4, 4096, 6144, 4
    inp = kda_inputs.conv_inputs(B=B, T=T, channels=Cn, K=K, dtype="bf16", seed=330, cache=False)
    x, w = inp["x"].cuda(), inp["weight"].cuda()
    out = torch.empty_like(x)
    fin = torch.empty((B, Cn, K - 1), dtype=torch.float32, device="cuda")

    def call():
        kda.short_conv(x, w, out=out, final_cache=fin)

    wall, ms = timed_calls(call, steps, warmup)
    avg = float(np.mean(ms))
    nb = conv_bytes(B * T, Cn, K, B)
    gbs = nb / (avg * 1e-3) / 1e9
    return {"workload": f"short causal depthwise conv, {B} x {T} tokens, {Cn} channels (q, k, v of 16 heads x 128), "
                        f"width {K}, bf16 in and out, zero caches",
            "tokens_per_s": round(B * T / (wall / steps), 1), "us_per_call": round(avg * 1e3, 2),
            "algorithmic_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}


def norm_bytes(rows: int, d: int, o_bytes=4, gate_bytes=2, out_bytes=2) -> int:
    """Algorithmic HBM bytes of one kda_gated_rmsnorm call: o and the gate read,
    out written once, the weight."""
    return rows * d * (o_bytes + gate_bytes + out_bytes) + d * 4


def bench_norm(kda, steps, warmup):
    """kda_gated_rmsnorm on the mixer output of the dense workload (4 x 4096
    tokens x 16 heads x 128: fp32 o, bf16 gate, bf16 out), timed like the
    prefill."""
    B, T, H, D = 4, 4096, 16, 128
    rng = np.random.default_rng(420)
    o = torch.from_numpy(rng.standard_normal((B, T, H, D), dtype=np.float32)).cuda()
    g = torch.from_numpy(rng.standard_normal((B, T, H, D), dtype=np.float32)).to(torch.bfloat16).cuda()
    w = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).cuda()
    out = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")

    def call():
        kda.gated_rmsnorm(o, g, w, 1e-6, out=out)

    wall, ms = timed_calls(call, steps, warmup)
    avg = float(np.mean(ms))
    nb = norm_bytes(B * T * H, D)
    gbs = nb / (avg * 1e-3) / 1e9
    return {"workload": f"gated per-head RMSNorm, {B} x {T} tokens x {H} heads x {D}, fp32 o, bf16 gate, bf16 out",
            "tokens_per_s": round(B * T / (wall / steps), 1), "us_per_call": round(avg * 1e3, 2),
            "algorithmic_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}


def bench_step(kda, name, steps, warmup):
    """kda_step timed per call with HIP events; before every call a 1 GiB
    buffer is read (clean lines, nothing to write back) so the state (128 MiB
    for verify) is not served from the 256 MB last-level cache left warm by
    the previous call."""
    inp = kda_inputs.config(name)
    d = to_dev(inp)
    N, n_tok, H, D = inp["q"].shape
    state = d["init_state"].clone()
    out = torch.empty((N, n_tok, H, D), dtype=torch.float32, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def call():
        kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, out=out)

    def flushed_call():
        torch.sum(flush, dim=0, out=sink)
        call()

    settle(flushed_call)
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(steps):
        torch.sum(flush, dim=0, out=sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    nbytes = step_bytes(N, n_tok, H, D)
    avg = float(np.mean(ms))
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"workload": f"{N} sequences x {n_tok} rows, H={H}, dk=dv={D}, bf16 q/k/v, fp32 state in place "
                        "(caches flushed before each call)",
            "us_per_call": round(avg * 1e3, 2), "achieved_GBs": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "algorithmic_bytes": nbytes}


def rows_bytes(N: int, n_tok: int, H: int, d: int, qkv_bytes=2) -> int:
    """kda_step_rows: the state read once (not written), each row in, its
    output and delta out."""
    per_row_head = 3 * d * qkv_bytes + d * 4 + 4 + d * 4 + d * 4
    return N * H * d * d * 4 + N * n_tok * H * per_row_head


def commit_bytes(N: int, n_tok: int, H: int, d: int, qkv_bytes=2) -> int:
    """kda_step_commit of every row: the state read and written, each row's
    k, log_g and delta read, the accept counts."""
    return N * H * 2 * d * d * 4 + N * n_tok * H * (d * qkv_bytes + d * 4 + d * 4) + N * 4


def bench_verify_commit(kda, steps, warmup):
    """Speculative verify on the verify workload: kda_step_rows (state read
    only) then kda_step_commit of all rows, each timed with HIP events after a
    1 GiB read, like bench_step."""
    inp = kda_inputs.config("verify")
    d = to_dev(inp)
    N, n_tok, H, D = inp["q"].shape
    state = d["init_state"].clone()
    out = torch.empty((N, n_tok, H, D), dtype=torch.float32, device="cuda")
    deltas = torch.empty((N, n_tok, H, D), dtype=torch.float32, device="cuda")
    accept = torch.full((N,), n_tok, dtype=torch.int32, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def rows():
        kda.step_rows(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, out=out, deltas=deltas)

    def commit():
        kda.step_commit(d["k"], d["log_g"], deltas, state, accept)

    def both():
        torch.sum(flush, dim=0, out=sink)
        rows()
        torch.sum(flush, dim=0, out=sink)
        commit()

    settle(both)
    for _ in range(warmup):
        both()
    stream = torch.cuda.current_stream()
    t_rows, t_commit = [], []
    for _ in range(steps):
        for fn, acc in ((rows, t_rows), (commit, t_commit)):
            torch.sum(flush, dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            acc.append(a.elapsed_time(b))
    r_us, c_us = float(np.mean(t_rows)) * 1e3, float(np.mean(t_commit)) * 1e3
    rb, cb = rows_bytes(N, n_tok, H, D), commit_bytes(N, n_tok, H, D)
    r_gbs, c_gbs = rb / (r_us * 1e-6) / 1e9, cb / (c_us * 1e-6) / 1e9
    roof = lambda g: {"bound": "hbm", "achieved": round(g, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(g / HBM_PEAK_GBS, 4), "traffic": None}
    return {"workload": f"{N} sequences x {n_tok} draft rows, H={H}, dk=dv={D}, bf16 q/k/v: rows scored with the "
                        "state read only, then every row committed (caches flushed before each call)",
            "rows": {"us_per_call": round(r_us, 2), "algorithmic_bytes": rb, "roofline": roof(r_gbs)},
            "commit": {"us_per_call": round(c_us, 2), "algorithmic_bytes": cb, "roofline": roof(c_gbs)}}


def cpu_baseline(inp, target_s=10.0):
    """Time the fp64 oracle on a bounded sample of the prefill workload: the
    whole workload (all sequences and heads, OpenMP over the units), repeated
    until about target_s of wall time has passed."""
    import oracle
    from kda_inputs import to_f64
    threads = max(1, min(16, os.cpu_count() or 1))
    B, T, H, D = inp["q"].shape
    args = (to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), to_f64(inp["log_g"]), to_f64(inp["beta"]))
    s0 = to_f64(inp["init_state"])
    reps, elapsed = 0, 0.0
    while elapsed < target_s:
        t0 = time.perf_counter()
        oracle.kda_forward(*args, init_state=s0, scale=inp["scale"], n_threads=threads)
        elapsed += time.perf_counter() - t0
        reps += 1
    token_heads = reps * B * T * H
    res = {"value": round(reps * B * T / elapsed, 1), "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"the whole workload ({B} x {T} tokens x {H} heads, fp64 token loop) run {reps} times "
                     f"back to back, {token_heads} token-heads in {elapsed:.1f} s on {threads} threads",
           "host_cpu": host_cpu_model()}
    # single-thread oracle on the small workloads (the whole of each, once)
    single = {}
    for name in ("tiny", "decode", "verify"):
        wi = kda_inputs.config(name)
        Nw, n_tok, Hw, Dw = wi["q"].shape
        st = to_f64(wi["init_state"]) if wi["init_state"] is not None else None
        t0 = time.perf_counter()
        oracle.kda_forward(to_f64(wi["q"]), to_f64(wi["k"]), to_f64(wi["v"]), to_f64(wi["log_g"]),
                           to_f64(wi["beta"]), init_state=st, scale=wi["scale"], n_threads=1)
        dt = time.perf_counter() - t0
        if name == "tiny":
            single[name] = {"tokens_per_s": round(Nw * n_tok / dt, 1)}
        else:
            single[name] = {"GB_per_s": round(step_bytes(Nw, n_tok, Hw, Dw) / dt / 1e9, 3)}
    res["single_thread"] = single
    return res


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_copy(steps, warmup):
    """A plain device copy of COPY_BYTES (the counter calibration kernel)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    wall, ms = timed_calls(lambda: dst.copy_(src), steps, warmup)
    avg = float(np.mean(ms))
    print(f"copy: {COPY_BYTES >> 20} MiB in {avg * 1e3:.1f} us = {2 * COPY_BYTES / (avg * 1e-3) / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "varlen", "step", "backward", "conv", "norm", "copy"],
                    default="all",
                    help="restrict the run (profiling); the JSON line needs 'all'")
    ap.add_argument("--traffic-from", nargs=4, metavar="DIR",
                    help="rocprofv3 csv dirs: FETCH_SIZE and WRITE_SIZE of the measured path, then FETCH_SIZE and "
                         "WRITE_SIZE of the copy; writes the path's profiles/traffic_*.txt")
    ap.add_argument("--traffic-kind", choices=sorted(TRAFFIC), default="prefill",
                    help="which path --traffic-from summarises (bench.py --only <kind> made its runs)")
    args = ap.parse_args()
    if args.traffic_from:
        kind = args.traffic_kind
        lines = write_traffic(*args.traffic_from, kind=kind)
        with open(TRAFFIC[kind]["file"], "w") as fh:
            fh.write(f"# HBM traffic of {TRAFFIC[kind]['what']}\n")
            fh.write(f"# made by: python bench.py --traffic-kind {kind} --traffic-from " + " ".join(args.traffic_from) + "\n")
            fh.write("# from four counter runs (cd /tmp && export TMPDIR=/tmp first), one pass each:\n")
            for ctr, what, d in (("FETCH_SIZE", kind, args.traffic_from[0]), ("WRITE_SIZE", kind, args.traffic_from[1]),
                                 ("FETCH_SIZE", "copy", args.traffic_from[2]), ("WRITE_SIZE", "copy", args.traffic_from[3])):
                steps = "--steps 3 --warmup 1"
                fh.write(f"#   rocprofv3 --pmc {ctr} -f csv -d {d} -o run -- python3 bench.py --only {what} {steps}\n")
            fh.write("# values are KiB per dispatch (mean over the run's dispatches); scale = copy bytes / counter bytes\n")
            fh.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import gated_delta_rule_67_amd as kda

    if args.only == "copy":
        bench_copy(args.steps, args.warmup)
        return
    res = {}
    if args.only in ("all", "prefill"):
        res["prefill"] = bench_prefill(kda, args.steps, args.warmup)
        print(f"prefill: mean {np.mean(res['prefill']['ms']) * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    if args.only in ("all", "varlen"):
        res["varlen"] = bench_varlen(kda, args.steps, args.warmup)
        print(f"varlen prefill: {res['varlen']['us_per_call']} us/call", file=sys.stderr, flush=True)
    if args.only in ("all", "backward"):
        res["backward"] = bench_backward(kda, args.steps, args.warmup)
        print(f"backward {res['backward']['us_per_call']} us per call", file=sys.stderr, flush=True)
    if args.only in ("all", "conv"):
        res["short_conv"] = bench_conv(kda, args.steps, args.warmup)
        print(f"short conv {res['short_conv']['us_per_call']} us per call", file=sys.stderr, flush=True)
    if args.only in ("all", "norm"):
        res["gated_rmsnorm"] = bench_norm(kda, args.steps, args.warmup)
        print(f"gated rmsnorm {res['gated_rmsnorm']['us_per_call']} us per call", file=sys.stderr, flush=True)
    if args.only in ("all", "step"):
        res["decode"] = bench_step(kda, "decode", args.steps, args.warmup)
        res["verify"] = bench_step(kda, "verify", args.steps, args.warmup)
        res["verify_rollback"] = bench_verify_commit(kda, args.steps, args.warmup)
        vr = res["verify_rollback"]
        print(f"decode {res['decode']['us_per_call']} us, verify {res['verify']['us_per_call']} us, "
              f"verify rows {vr['rows']['us_per_call']} us + commit {vr['commit']['us_per_call']} us",
              file=sys.stderr, flush=True)
    if args.only != "all":
        return

    p = res["prefill"]
    ms_per_step = p["wall"] / args.steps * 1e3
    value = p["tokens"] / (ms_per_step * 1e-3)
    k_ms = float(np.mean(p["ms"]))
    gbs = p["bytes"] / (k_ms * 1e-3) / 1e9
    tflops = p["flops"] / (k_ms * 1e-3) / 1e12
    line = {
        "metric": "KDA prefill tokens/s (+MFMA %) and decode state-update HBM GB/s, dk=dv=128",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands, f32 accumulation and state (bf16 inputs)",
        "data": "synthetic (seeded; q,v~N(0,1), k L2-normalised, log_g=-softplus(N)*0.05, beta=sigmoid(N))",
        "config": {"workload": "chunked prefill, dense B=4 x T=4096, H=16, dk=dv=128, bf16 q/k/v, "
                               "fp32 log_g/beta/state, fp32 out, chunk 64",
                   "global_batch": 4, "seq_len": 4096, "heads": 16, "head_dim": 128},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                     "kernel": "kda_chunk_fwd = prep_kernel + scan_kernel back to back (one call)"},
        "prefill_kernel_us": round(k_ms * 1e3, 2),
        "algorithmic_bytes_per_launch": p["bytes"],
        "mfma": {"achieved_TFLOPs": round(tflops, 2), "peak_TFLOPs": MFMA_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "algorithmic_flop_per_launch": p["flops"]},
        "varlen": res["varlen"],
        "decode": res["decode"],
        "verify": res["verify"],
        "verify_rollback": res["verify_rollback"],
        "backward": res["backward"],
        "short_conv": res["short_conv"],
        "gated_rmsnorm": res["gated_rmsnorm"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p["inp"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
