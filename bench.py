"""Benchmark of libkda on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --only {prefill,varlen,step,backward,conv,norm,strong,copy,peak}   (profiling runs)
    python bench.py [--traffic-kind KIND] --traffic-from FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
    python bench.py --mfma-from SQ_DIR                                      (MFMA counter summary)

A step is one kda_chunk_fwd call (chunked prefill) over the packed workload:
one row of 65536 tokens split into 26 documents of log-uniform length
(64..16384), H=32 heads, dk=dv=128, bf16 q/k/v, fp32 gates/beta, zero initial
states, fp32 out and final states, inputs resident in HBM.  ``value`` is its
tokens/s over exactly K back-to-back calls (wall clock between two
synchronisations).  The same JSON line carries:
  roofline      that call: algorithmic bytes per call / mean call time (one
                HIP event pair on the launch stream around the K calls)
                against 8 TB/s HBM, with the counter-measured traffic
  flushed       the same call timed one by one after a 1 GiB read that evicts
                the last-level cache: median / p10 / p90 over 100 calls
  mfma          algorithmic FLOP/s against the 2516.6 TFLOP/s dense 16-bit
                MFMA peak, and the counter-measured MFMA busy fraction
  dense_prefill the dense 4 x 4096-token, 16-head prefill, timed the same ways
  strong_gates  the dense workload with stronger gates (log_g scale 1.0 and
                log_g ~ U[-5, 0]): tokens/s and the fraction of chunks that
                take the exact per-token fallback instead of the MFMA path
  decode/verify kda_step on 256 x 1 and 64 x 4 rows, H=32, d=128, each with
                its own HBM roofline (state read + write + row traffic)
  verify_rollback  the 64 x 4-row verify split into kda_step_rows and
                kda_step_commit, each with its own HBM roofline
  backward      kda_chunk_bwd on the dense workload (fp32 matrix-core roofline)
  short_conv, gated_rmsnorm   the two elementwise kernels' HBM rooflines
  peaks         this GPU's re-measured peaks: a plain 1 GiB device copy (GB/s)
                and a dense fp16 MFMA loop (TFLOP/s), against which the
                rooflines above can also be read
  cpu_baseline  the fp64 oracle timed on the host on a bounded sample
Every timed region follows SETTLE_S seconds of the same workload run back to
back (untimed), then the W warm-up steps: the GPU's clocks need some 30 ms
of sustained load to reach their steady state.
Only one GPU is used; --gpus above 1 exits with a message.

Counter summaries under profiles/ (HBM traffic from FETCH_SIZE / WRITE_SIZE,
scaled by what the same counters read for a plain copy of known size; MFMA
busy cycles) are stamped with a hash of the kernel sources and reported only
while the sources still hash the same (else null).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
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
    "varlen": dict(file=os.path.join(ROOT, "profiles", "traffic_prefill_packed.txt"),
                   sources=["kda_twopass.hip", "kda_common.h", "kda_fallback.h"],
                   kernels=("prep_kernel", "scan_kernel", "scan4_kernel"),
                   what="one kda_chunk_fwd call, packed 65536 tokens in 26 documents, 32 heads, d = 128, bf16"),
    "prefill": dict(file=os.path.join(ROOT, "profiles", "traffic_prefill_dense.txt"),
                    sources=["kda_twopass.hip", "kda_common.h", "kda_fallback.h"],
                    kernels=("prep_kernel", "scan_kernel", "scan4_kernel"),
                    what="one kda_chunk_fwd call, dense 4 x 4096 tokens, 16 heads, d = 128, bf16"),
    "backward": dict(file=os.path.join(ROOT, "profiles", "traffic_backward_dense.txt"),
                     sources=["kda_backward.hip", "kda_common.h"],
                     kernels=("bwd_prep", "bwd_fscan", "bwd_rscan", "bwd_gstate", "bwd_gpairs"),
                     what="one kda_chunk_bwd call, dense 4 x 4096 tokens, 16 heads, d = 128, bf16"),
    # the decode dispatches only: the whole-tile instantiation at 256 x 32
    # units of 512 threads (verify's one-row reference uses it at 64 x 32
    # units; verify and the speculative rows use the half-width one); its
    # counter runs are bench.py --only step
    "decode": dict(file=os.path.join(ROOT, "profiles", "traffic_decode.txt"),
                   sources=["kda_recurrent.hip", "kda_common.h"],
                   kernels=("recurrent_kernel<128, 128",), only="step", grid=256 * 32 * 512,
                   what="one kda_step decode call, 256 sequences x 1 row, 32 heads, d = 128, bf16 q/k/v, "
                        "fp32 state in place, caches flushed before each call"),
}
# MFMA counter summaries, one per prefill workload (the counter run is
# bench.py --only <kind>)
MFMA = {
    "varlen": dict(file=os.path.join(ROOT, "profiles", "mfma_prefill_packed.txt"),
                   what="one kda_chunk_fwd call, packed 65536 tokens in 26 documents, 32 heads, d = 128, bf16"),
    "prefill": dict(file=os.path.join(ROOT, "profiles", "mfma_prefill_dense.txt"),
                    what="one kda_chunk_fwd call, dense 4 x 4096 tokens, 16 heads, d = 128, bf16"),
}


def code_only(text: str) -> str:
    """C++ source with comments and blank lines removed and line ends
    trimmed: the part of a kernel source that decides what the counters
    measure (string literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def sources_hash(kind: str = "prefill") -> str:
    """Hash of the code (comments aside) of the sources that define a measured
    path's kernels; a counter summary is used only while it matches."""
    h = hashlib.sha256()
    for f in TRAFFIC[kind]["sources"]:
        with open(os.path.join(ROOT, "gated_delta_rule_67_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
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


def _counter_sums(run_dir: str, counter: str, grid=None):
    """{kernel name: mean per-dispatch value} of one rocprofv3 --pmc csv run;
    with grid, only the dispatches of that many threads."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            if grid is not None and int(r["Grid_Size"]) != grid:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in out.items()}


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kind="prefill"):
    grid = TRAFFIC[kind].get("grid")
    fe, wr = _counter_sums(fetch_dir, "FETCH_SIZE", grid), _counter_sums(write_dir, "WRITE_SIZE", grid)
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
    synchronisation.  Returns (wall seconds of the timed region, mean event
    milliseconds per call).  One pair of HIP events on the launch stream spans
    the steps calls: an event recorded between two calls holds the next
    call's first kernel back until the event has been signalled, a gap the
    calls themselves do not have."""
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
    return wall, a.elapsed_time(b) / steps


class CacheFlush:
    """Reads a 1 GiB buffer: the lines it leaves in the 256 MB last-level
    cache are clean, so the next call neither hits on its own inputs nor pays
    a write-back."""

    def __init__(self):
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        torch.sum(self.buf, dim=0, out=self.sink)


def flushed_calls(fn, n: int, flush: CacheFlush):
    """fn timed n times one by one with HIP events on the launch stream, the
    cache flushed before each call.  Returns the per-call milliseconds."""
    def one():
        flush()
        fn()
    settle(one)
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(n):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    return ms


def spread(ms, back_to_back_ms=None):
    """median / p10 / p90 of per-call milliseconds, in microseconds."""
    x = np.asarray(ms, dtype=np.float64) * 1e3
    r = {"n": int(x.size), "median_us": round(float(np.median(x)), 2),
         "p10_us": round(float(np.percentile(x, 10)), 2), "p90_us": round(float(np.percentile(x, 90)), 2)}
    if back_to_back_ms is not None:
        r["back_to_back_mean_us"] = round(back_to_back_ms * 1e3, 2)
    return r


def to_dev(inp):
    return {k: (inp[k].cuda().contiguous() if inp[k] is not None else None)
            for k in ("q", "k", "v", "log_g", "beta", "init_state", "cu_seqlens")}


def hbm_roofline(nbytes: int, ms: float, traffic=None, **extra):
    gbs = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    r.update(extra)
    return r


def bench_prefill_workload(kda, name, steps, warmup, flush, n_flushed=100, **overrides):
    """One prefill workload (dense or packed, kda_inputs config ``name``): K
    back-to-back calls (wall clock and one event pair), then ``n_flushed``
    calls one by one after a cache flush."""
    inp = kda_inputs.config(name, **overrides)
    d = to_dev(inp)
    B, T, H, D = inp["q"].shape
    packed = d["cu_seqlens"] is not None
    N = d["cu_seqlens"].numel() - 1 if packed else B
    out = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(N, T, H, D, packed=packed), dtype=torch.uint8, device="cuda")

    def call():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"],
                      cu_seqlens=d["cu_seqlens"], out=out, final_state=fin, workspace=ws)

    wall, mean_ms = timed_calls(call, steps, warmup)
    flushed = flushed_calls(call, n_flushed, flush) if n_flushed else None
    tokens = B * T
    n_states = N if inp["init_state"] is not None else 0
    nbytes = prefill_bytes(tokens, H, D, n_states=n_states) + N * H * D * D * 4 * (n_states == 0)
    return dict(inp=inp, wall=wall, mean_ms=mean_ms, flushed=flushed, tokens=tokens, N=N, H=H, D=D,
                packed=packed, bytes=nbytes, flops=prefill_flops(tokens, H, D), ws_bytes=int(ws.numel()),
                call=call, d=d, ws=ws)


def prefill_summary(p, steps, traffic=None, kernel=None):
    """The reported object of one prefill workload."""
    tf = p["flops"] / (p["mean_ms"] * 1e-3) / 1e12
    r = {"tokens_per_s": round(p["tokens"] / (p["wall"] / steps), 1),
         "token_heads_per_s": round(p["tokens"] * p["H"] / (p["wall"] / steps), 1),
         "us_per_call": round(p["mean_ms"] * 1e3, 2),
         "algorithmic_bytes": p["bytes"], "algorithmic_flops": p["flops"],
         "roofline": hbm_roofline(p["bytes"], p["mean_ms"], traffic,
                                  **({"kernel": kernel} if kernel else {})),
         "mfma": {"achieved_TFLOPs": round(tf, 2), "peak_TFLOPs": MFMA_PEAK_TFLOPS,
                  "frac": round(tf / MFMA_PEAK_TFLOPS, 4)},
         "workspace_bytes": p["ws_bytes"]}
    if p["flushed"]:
        r["flushed"] = spread(p["flushed"], p["mean_ms"])
    return r


SLOT_BYTES, SLOT_FLAG_OFF = 74752, 74240  # workspace slot of one (chunk, head); its per-wave fallback bytes


def tree_fraction(inp) -> float:
    """Fraction of (chunk, head) pairs whose diagonal tiles the prep kernel
    builds from the binary pair tree (decay beyond e^-6 over the first or the
    second half of any 16-token block, in any channel), computed on the host
    from log_g."""
    g = inp["log_g"].double().numpy()
    B, T, H, D = g.shape
    nch = (T + CHUNK - 1) // CHUNK
    pad = nch * CHUNK - T
    if pad:
        g = np.concatenate([g, np.zeros((B, pad, H, D))], axis=1)
    half = g.reshape(B, nch, 4, 2, 8, H, D).sum(axis=4)  # [B, chunk, block, half, H, D]
    return float((half < -6.0).any(axis=(2, 3, 5)).mean())


def fallback_fraction(ws, n_slots: int) -> float:
    """Fraction of (chunk, head) slots the prep kernel flagged for the exact
    per-token fallback, read from the flags it wrote into a dense problem's
    workspace (the scan's own state and Delta bounds are not included)."""
    flags = ws[: n_slots * SLOT_BYTES].view(n_slots, SLOT_BYTES)[:, SLOT_FLAG_OFF:SLOT_FLAG_OFF + 8]
    return float((flags != 0).any(dim=1).float().mean())


def bench_strong_gates(kda, steps, warmup, flush):
    """The dense workload with stronger gates than its 0.05 scale: log_g =
    -softplus(N(0,1)) at scale 1.0, and log_g ~ U[-5, 0].  Reports tokens/s,
    the fraction of (chunk, head) pairs whose diagonal tiles come from the
    pair tree, and the fraction the prep kernel sent to the exact per-token
    fallback."""
    res = {}
    for tag, over in (("gate_scale_1.0", dict(gate_scale=1.0)), ("uniform_-5_0", dict(gate_uniform=5.0))):
        p = bench_prefill_workload(kda, "prefill", steps, warmup, flush, n_flushed=0, **over)
        B, T, H = p["inp"]["q"].shape[:3]
        res[tag] = {"tokens_per_s": round(p["tokens"] / (p["wall"] / steps), 1),
                    "us_per_call": round(p["mean_ms"] * 1e3, 2),
                    "tree_chunk_fraction": round(tree_fraction(p["inp"]), 4),
                    "fallback_chunk_fraction": round(fallback_fraction(p["ws"], B * ((T + CHUNK - 1) // CHUNK) * H),
                                                     4)}
        del p
        torch.cuda.empty_cache()
    return res


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

    wall, avg = timed_calls(call, steps, warmup)
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

    wall, avg = timed_calls(call, steps, warmup)
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

    wall, avg = timed_calls(call, steps, warmup)
    nb = norm_bytes(B * T * H, D)
    gbs = nb / (avg * 1e-3) / 1e9
    return {"workload": f"gated per-head RMSNorm, {B} x {T} tokens x {H} heads x {D}, fp32 o, bf16 gate, bf16 out",
            "tokens_per_s": round(B * T / (wall / steps), 1), "us_per_call": round(avg * 1e3, 2),
            "algorithmic_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}


def bench_fused_norm(kda, steps, warmup):
    """The mixer's output path on the dense and packed workloads, bf16 out,
    three ways, timed like the prefill: kda_chunk_fwd_gated_norm (the norm in
    the scan's epilogue, one call); kda_chunk_fwd with fp32 out followed by
    kda_gated_rmsnorm (the two calls it replaces); kda_chunk_fwd with bf16 out
    and no norm (the floor of the pair)."""
    res = {}
    for name in ("prefill", "varlen"):
        inp = kda_inputs.config(name)
        d = to_dev(inp)
        B, T, H, D = inp["q"].shape
        packed = d["cu_seqlens"] is not None
        N = d["cu_seqlens"].numel() - 1 if packed else B
        rng = np.random.default_rng(421)
        g = torch.from_numpy(rng.standard_normal((B, T, H, D), dtype=np.float32)).to(torch.bfloat16).cuda()
        w = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).cuda()
        o32 = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
        o16 = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
        fin = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(kda.workspace_bytes(N, T, H, D, packed=packed), dtype=torch.uint8, device="cuda")
        kw = dict(init_state=d["init_state"], cu_seqlens=d["cu_seqlens"], final_state=fin, workspace=ws)
        args = (d["q"], d["k"], d["v"], d["log_g"], d["beta"])

        def fused():
            kda.chunk_fwd_gated_norm(*args, g, w, 1e-6, out=o16, **kw)

        def two_calls():
            kda.chunk_fwd(*args, out=o32, **kw)
            kda.gated_rmsnorm(o32, g, w, 1e-6, out=o16)

        def plain_bf16():
            kda.chunk_fwd(*args, out=o16, out_dtype=torch.bfloat16, **kw)

        r = {}
        for tag, fn in (("fused_gated_norm", fused), ("chunk_fwd_then_norm", two_calls),
                        ("chunk_fwd_bf16_no_norm", plain_bf16)):
            _, ms = timed_calls(fn, steps, warmup)
            r[tag + "_us"] = round(ms * 1e3, 2)
        res[name] = r
        del d, g, o32, o16, fin, ws
        torch.cuda.empty_cache()
    return res


def bench_step(kda, name, steps, warmup, flush):
    """kda_step timed per call with HIP events; before every call a 1 GiB
    buffer is read (clean lines, nothing to write back) so the state (128 MiB
    for verify) is not served from the 256 MB last-level cache left warm by
    the previous call.  Reports the mean and the median / p10 / p90."""
    inp = kda_inputs.config(name)
    d = to_dev(inp)
    N, n_tok, H, D = inp["q"].shape
    state = d["init_state"].clone()
    out = torch.empty((N, n_tok, H, D), dtype=torch.float32, device="cuda")

    def call():
        kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, out=out)

    for _ in range(warmup):
        call()
    ms = flushed_calls(call, max(steps, 100), flush)
    nbytes = step_bytes(N, n_tok, H, D)
    avg = float(np.mean(ms))
    r = {"workload": f"{N} sequences x {n_tok} rows, H={H}, dk=dv={D}, bf16 q/k/v, fp32 state in place "
                     "(caches flushed before each call)",
         "us_per_call": round(avg * 1e3, 2), "achieved_GBs": round(nbytes / (avg * 1e-3) / 1e9, 1),
         "per_call": spread(ms),
         "roofline": hbm_roofline(nbytes, avg, traffic=read_traffic("decode") if name == "decode" else None),
         "algorithmic_bytes": nbytes}
    if n_tok > 1:
        # the same states streamed by a one-row step: what the state traffic
        # alone reaches at this many units
        q1 = {k: d[k][:, :1].contiguous() for k in ("q", "k", "v", "log_g", "beta")}
        out1 = torch.empty((N, 1, H, D), dtype=torch.float32, device="cuda")

        def call1():
            kda.step(q1["q"], q1["k"], q1["v"], q1["log_g"], q1["beta"], state, out=out1)

        ms1 = flushed_calls(call1, max(steps, 100), flush)
        nb1 = step_bytes(N, 1, H, D)
        a1 = float(np.mean(ms1))
        r["one_row_same_states"] = {"us_per_call": round(a1 * 1e3, 2),
                                    "achieved_GBs": round(nb1 / (a1 * 1e-3) / 1e9, 1),
                                    "algorithmic_bytes": nb1}
    return r


def rows_bytes(N: int, n_tok: int, H: int, d: int, qkv_bytes=2) -> int:
    """kda_step_rows: the state read once (not written), each row in, its
    output and delta out."""
    per_row_head = 3 * d * qkv_bytes + d * 4 + 4 + d * 4 + d * 4
    return N * H * d * d * 4 + N * n_tok * H * per_row_head


def commit_bytes(N: int, n_tok: int, H: int, d: int, qkv_bytes=2) -> int:
    """kda_step_commit of every row: the state read and written, each row's
    k, log_g and delta read, the accept counts."""
    return N * H * 2 * d * d * 4 + N * n_tok * H * (d * qkv_bytes + d * 4 + d * 4) + N * 4


def bench_verify_commit(kda, steps, warmup, flush):
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

    def rows():
        kda.step_rows(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, out=out, deltas=deltas)

    def commit():
        kda.step_commit(d["k"], d["log_g"], deltas, state, accept)

    for _ in range(warmup):
        rows()
        commit()
    n = max(steps, 100)
    t_rows = flushed_calls(rows, n, flush)
    t_commit = flushed_calls(commit, n, flush)
    r_ms, c_ms = float(np.mean(t_rows)), float(np.mean(t_commit))
    rb, cb = rows_bytes(N, n_tok, H, D), commit_bytes(N, n_tok, H, D)
    return {"workload": f"{N} sequences x {n_tok} draft rows, H={H}, dk=dv={D}, bf16 q/k/v: rows scored with the "
                        "state read only, then every row committed (caches flushed before each call)",
            "rows": {"us_per_call": round(r_ms * 1e3, 2), "per_call": spread(t_rows), "algorithmic_bytes": rb,
                     "roofline": hbm_roofline(rb, r_ms)},
            "commit": {"us_per_call": round(c_ms * 1e3, 2), "per_call": spread(t_commit), "algorithmic_bytes": cb,
                       "roofline": hbm_roofline(cb, c_ms)}}


def host_cores():
    """(threads the oracle runs on, logical CPUs this process may use, nproc).
    The oracle uses the CPUs this process may run on, capped by
    OMP_NUM_THREADS when the environment sets it (a GPU host grants each GPU
    a share of its cores and says so there)."""
    nproc = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = nproc
    threads = allowed
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    return max(1, threads), allowed, nproc


def host_cpu_model() -> str:
    """lscpu's model name (else /proc/cpuinfo's)."""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, ValueError, Exception):  # noqa: BLE001 - best effort description
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, target_s=10.0):
    """Time the fp64 oracle on a bounded sample of the headline workload: the
    whole packed workload (all documents and heads, OpenMP over the units,
    longest first), repeated until about target_s of wall time has passed."""
    import oracle
    from kda_inputs import to_f64
    threads, allowed, nproc = host_cores()
    B, T, H, D = inp["q"].shape
    args = (to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), to_f64(inp["log_g"]), to_f64(inp["beta"]))
    cu = inp["cu_seqlens"].numpy().astype(np.int64) if inp["cu_seqlens"] is not None else None
    s0 = to_f64(inp["init_state"])
    reps, elapsed = 0, 0.0
    while elapsed < target_s:
        t0 = time.perf_counter()
        oracle.kda_forward(*args, init_state=s0, cu_seqlens=cu, scale=inp["scale"], n_threads=threads)
        elapsed += time.perf_counter() - t0
        reps += 1
    token_heads = reps * B * T * H
    res = {"value": round(reps * B * T / elapsed, 1), "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"the whole packed workload ({B} x {T} tokens, {H} heads, fp64 token loop) run {reps} times "
                     f"back to back, {token_heads} token-heads in {elapsed:.1f} s on {threads} threads",
           "host_cpu": host_cpu_model(), "nproc": nproc, "cpus_allowed": allowed,
           "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    del args
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


PEAK_LIB = os.path.join(ROOT, "gated_delta_rule_67_amd", "libkda_peak.so")


def bench_peaks(steps, warmup):
    """This GPU's re-measured peaks: a 1 GiB device-to-device copy (bytes read
    plus written per second) and the dense fp16 MFMA loop of libkda_peak.so."""
    import ctypes
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    _, ms = timed_calls(lambda: dst.copy_(src), steps, warmup)
    copy_gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst
    lib = ctypes.CDLL(PEAK_LIB)
    lib.kda_peak_mfma_f16.restype = ctypes.c_int
    lib.kda_peak_mfma_f16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, iters = 2048, 4000
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def mfma():
        rc = lib.kda_peak_mfma_f16(blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"kda_peak_mfma_f16 failed ({rc})")

    _, ms = timed_calls(mfma, max(3, steps // 4), 1)
    flop = blocks * 4 * iters * 8 * 16384
    tf = flop / (ms * 1e-3) / 1e12
    return {"copy_GBs": round(copy_gbs, 1), "copy_frac_of_8TBs": round(copy_gbs / HBM_PEAK_GBS, 4),
            "mfma_f16_TFLOPs": round(tf, 1), "mfma_frac_of_2516TF": round(tf / MFMA_PEAK_TFLOPS, 4),
            "how": "copy: torch copy_ of 1 GiB fp32 (read + write); mfma: 2048 workgroups x 4 waves x 4000 "
                   "rounds of 8 independent v_mfma_f32_16x16x32_f16"}


def bench_copy(steps, warmup):
    """A plain device copy of COPY_BYTES (the counter calibration kernel)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    _, ms = timed_calls(lambda: dst.copy_(src), steps, warmup)
    print(f"copy: {COPY_BYTES >> 20} MiB in {ms * 1e3:.1f} us = {2 * COPY_BYTES / (ms * 1e-3) / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)


# rocprofv3's derived MFMA metrics (it applies their reductions over SIMDs and
# XCDs): MfmaUtil = 100 * sum SQ_VALU_MFMA_BUSY_CYCLES / (max GRBM_GUI_ACTIVE *
# SIMD_NUM); MfmaFlopsF16 = 512 * SQ_INSTS_VALU_MFMA_MOPS_F16.  One pass.
MFMA_COUNTERS = ("MfmaUtil", "MfmaFlopsF16")


def write_mfma(run_dir, kind="varlen"):
    """Per-kernel MFMA metrics of one rocprofv3 --pmc run (mean per dispatch):
    the busy fraction of the matrix cores while the kernel runs, and the fp16
    MFMA FLOP it executed (algorithmic plus any redundant work)."""
    lines = [f"sources_sha256: {sources_hash(kind)}"]
    per = {}
    for c in MFMA_COUNTERS:
        try:
            per[c] = _counter_sums(run_dir, c)
        except SystemExit:
            per[c] = {}
    for pat in TRAFFIC[kind]["kernels"]:
        util = [v for k, v in per["MfmaUtil"].items() if pat in k]
        flop = sum(v for k, v in per["MfmaFlopsF16"].items() if pat in k)
        if util:
            lines.append(f"{pat}_mfma_busy_frac: {util[0] / 100.0:.4f}")
        lines.append(f"{pat}_counted_mfma_flop: {flop:.0f}")
    return lines


def read_mfma(kind="varlen"):
    """The committed MFMA counter summary of a prefill workload as a dict, or
    None when it is missing or was taken on other kernel sources."""
    try:
        kv = {}
        for line in open(MFMA[kind]["file"]):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.pop("sources_sha256", None) != sources_hash(kind):
            return None
        return {k: float(v) for k, v in kv.items()}
    except (OSError, ValueError):
        return None


def add_mfma_counters(summary, p, kind):
    """Counted MFMA FLOP per call, their rate against the fp16 peak, and each
    kernel's busy fraction, from the committed summary of this workload."""
    mf = read_mfma(kind)
    if mf is None:
        return
    counted = sum(mf.get(f"{k}_counted_mfma_flop", 0.0) for k in TRAFFIC[kind]["kernels"])
    summary["mfma"]["counted_mfma_flop_per_call"] = counted
    summary["mfma"]["counted_TFLOPs"] = round(counted / (p["mean_ms"] * 1e-3) / 1e12, 2)
    summary["mfma"]["counted_frac"] = round(counted / (p["mean_ms"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)
    summary["mfma"]["busy_frac"] = {k: mf[f"{k}_mfma_busy_frac"] for k in TRAFFIC[kind]["kernels"]
                                    if f"{k}_mfma_busy_frac" in mf}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "varlen", "step", "backward", "conv", "norm", "strong",
                                       "copy", "peak"],
                    default="all", help="restrict the run (profiling); the JSON line needs 'all'")
    ap.add_argument("--traffic-from", nargs=4, metavar="DIR",
                    help="rocprofv3 csv dirs: FETCH_SIZE and WRITE_SIZE of the measured path, then FETCH_SIZE and "
                         "WRITE_SIZE of the copy; writes the path's profiles/traffic_*.txt")
    ap.add_argument("--traffic-kind", choices=sorted(TRAFFIC), default="varlen",
                    help="which path --traffic-from summarises (bench.py --only <kind> made its runs)")
    ap.add_argument("--mfma-from", metavar="DIR",
                    help="rocprofv3 csv dir of one --pmc run of the MFMA counters over --only <--mfma-kind>; "
                         "writes that workload's profiles/mfma_prefill_*.txt")
    ap.add_argument("--mfma-kind", choices=sorted(MFMA), default="varlen")
    args = ap.parse_args()
    if args.traffic_from:
        kind = args.traffic_kind
        lines = write_traffic(*args.traffic_from, kind=kind)
        with open(TRAFFIC[kind]["file"], "w") as fh:
            fh.write(f"# HBM traffic of {TRAFFIC[kind]['what']}\n")
            fh.write(f"# made by: python bench.py --traffic-kind {kind} --traffic-from " + " ".join(args.traffic_from) + "\n")
            fh.write("# from four counter runs (cd /tmp && export TMPDIR=/tmp first), one pass each:\n")
            only = TRAFFIC[kind].get("only", kind)
            for ctr, what, d in (("FETCH_SIZE", only, args.traffic_from[0]), ("WRITE_SIZE", only, args.traffic_from[1]),
                                 ("FETCH_SIZE", "copy", args.traffic_from[2]), ("WRITE_SIZE", "copy", args.traffic_from[3])):
                steps = "--steps 3 --warmup 1"
                fh.write(f"#   rocprofv3 --pmc {ctr} -f csv -d {d} -o run -- python3 bench.py --only {what} {steps}\n")
            grid = TRAFFIC[kind].get("grid")
            fh.write("# values are KiB per dispatch (mean over the run's dispatches"
                     + (f" of {grid} threads" if grid else "") + "); scale = copy bytes / counter bytes\n")
            fh.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if args.mfma_from:
        kind = args.mfma_kind
        lines = write_mfma(args.mfma_from, kind)
        with open(MFMA[kind]["file"], "w") as fh:
            fh.write(f"# MFMA counters of {MFMA[kind]['what']}\n")
            fh.write(f"# made by: python bench.py --mfma-kind {kind} --mfma-from {args.mfma_from}\n")
            fh.write(f"# from: rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} -f csv -d {args.mfma_from} -o run -- "
                     f"python3 bench.py --only {kind} --steps 3 --warmup 1\n")
            fh.write("# values are per dispatch (mean over the run's dispatches); mfma_busy_frac = MfmaUtil / 100 "
                     "(busy cycles of the matrix cores over the kernel's active cycles on all SIMDs); "
                     "counted_mfma_flop = MfmaFlopsF16\n")
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
    flush = CacheFlush()
    res = {}
    if args.only in ("all", "varlen"):
        res["varlen"] = bench_prefill_workload(kda, "varlen", args.steps, args.warmup, flush,
                                               n_flushed=100 if args.only == "all" else 0)
        print(f"packed prefill: {res['varlen']['mean_ms'] * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    if args.only in ("all", "prefill"):
        res["prefill"] = bench_prefill_workload(kda, "prefill", args.steps, args.warmup, flush,
                                                n_flushed=100 if args.only == "all" else 0)
        print(f"dense prefill: {res['prefill']['mean_ms'] * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    if args.only in ("all", "strong"):
        res["strong_gates"] = bench_strong_gates(kda, args.steps, args.warmup, flush)
        print(f"strong gates: {res['strong_gates']}", file=sys.stderr, flush=True)
    if args.only in ("all", "backward"):
        res["backward"] = bench_backward(kda, args.steps, args.warmup)
        print(f"backward {res['backward']['us_per_call']} us per call", file=sys.stderr, flush=True)
    if args.only in ("all", "conv"):
        res["short_conv"] = bench_conv(kda, args.steps, args.warmup)
        print(f"short conv {res['short_conv']['us_per_call']} us per call", file=sys.stderr, flush=True)
    if args.only in ("all", "norm"):
        res["gated_rmsnorm"] = bench_norm(kda, args.steps, args.warmup)
        print(f"gated rmsnorm {res['gated_rmsnorm']['us_per_call']} us per call", file=sys.stderr, flush=True)
        res["fused_gated_norm"] = bench_fused_norm(kda, args.steps, args.warmup)
        print(f"fused gated norm {res['fused_gated_norm']}", file=sys.stderr, flush=True)
    if args.only in ("all", "step"):
        res["decode"] = bench_step(kda, "decode", args.steps, args.warmup, flush)
        res["verify"] = bench_step(kda, "verify", args.steps, args.warmup, flush)
        res["verify_rollback"] = bench_verify_commit(kda, args.steps, args.warmup, flush)
        vr = res["verify_rollback"]
        print(f"decode {res['decode']['us_per_call']} us, verify {res['verify']['us_per_call']} us, "
              f"verify rows {vr['rows']['us_per_call']} us + commit {vr['commit']['us_per_call']} us",
              file=sys.stderr, flush=True)
    if args.only in ("all", "peak"):
        res["peaks"] = bench_peaks(args.steps, args.warmup)
        print(f"peaks {res['peaks']}", file=sys.stderr, flush=True)
    if args.only != "all":
        return

    p = res["varlen"]
    ms_per_step = p["wall"] / args.steps * 1e3
    value = p["tokens"] / (ms_per_step * 1e-3)
    head = prefill_summary(p, args.steps, read_traffic("varlen"),
                           kernel="kda_chunk_fwd = prep_kernel + scan4_kernel back to back (one call)")
    add_mfma_counters(head, p, "varlen")
    dense = prefill_summary(res["prefill"], args.steps, read_traffic("prefill"))
    add_mfma_counters(dense, res["prefill"], "prefill")
    dense["workload"] = ("chunked prefill, dense B=4 x T=4096, H=16, dk=dv=128, bf16 q/k/v, fp32 log_g/beta/"
                         "state, fp32 out, chunk 64")
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
        "dtype": "bf16 in; f16 MFMA operands, f32 accumulation, state and out",
        "data": "synthetic (seeded; q,v~N(0,1), k L2-normalised, log_g=-softplus(N)*0.05, beta=sigmoid(N))",
        "config": {"workload": f"packed varlen chunked prefill: 1 x {p['tokens']} tokens in {p['N']} documents "
                               "(log-uniform 64..16384), H=32, dk=dv=128, bf16 q/k/v, fp32 log_g/beta, zero initial "
                               "states, fp32 out and final states, chunk 64",
                   "global_batch": 1, "seq_len": p["tokens"], "documents": p["N"], "heads": 32, "head_dim": 128},
        "roofline": head["roofline"],
        "flushed": head["flushed"],
        "prefill_kernel_us": head["us_per_call"],
        "algorithmic_bytes_per_launch": p["bytes"],
        "mfma": dict(head["mfma"], algorithmic_flop_per_launch=p["flops"]),
        "token_heads_per_s": head["token_heads_per_s"],
        "dense_prefill": dense,
        "strong_gates": res["strong_gates"],
        "decode": res["decode"],
        "verify": res["verify"],
        "verify_rollback": res["verify_rollback"],
        "backward": res["backward"],
        "short_conv": res["short_conv"],
        "gated_rmsnorm": res["gated_rmsnorm"],
        "fused_gated_norm": res["fused_gated_norm"],
        "peaks": res["peaks"],
    }
    inp = p["inp"]
    for k in list(res):
        res[k] = None
    del p
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
