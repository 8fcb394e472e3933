"""Benchmark of libkda on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one kda_chunk_fwd call (chunked prefill) over the dense workload
B=4 x T=4096 tokens, H=16 heads, dk=dv=128, bf16 q/k/v, fp32 gates/beta/state,
fp32 out, with inputs resident in HBM.  ``value`` is prefill tokens/s
(tokens of the 16-head mixer per second).  The same JSON line carries:
  roofline      prefill kernel: algorithmic bytes per launch / mean launch time
                (HIP events on the launch stream) against 8 TB/s HBM
  mfma          algorithmic prefill FLOP/s against the 2516.6 TFLOP/s dense
                16-bit MFMA peak
  decode/verify kda_step GB/s on 256 x 1 and 64 x 4 rows, H=32, d=128, each
                with its own roofline (state read + write + row traffic)
  cpu_baseline  the fp64 oracle timed on the host on a bounded sample of the
                same prefill workload
Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
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
CHUNK = 64


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


def timed_calls(fn, steps: int, warmup: int):
    """Run fn warmup times, then steps times bracketed by synchronisation.
    Returns (wall seconds of the timed region, per-call event milliseconds)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in ev]


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


def bench_step(kda, name, steps, warmup):
    inp = kda_inputs.config(name)
    d = to_dev(inp)
    N, n_tok, H, D = inp["q"].shape
    state = d["init_state"].clone()
    out = torch.empty((N, n_tok, H, D), dtype=torch.float32, device="cuda")

    def call():
        kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, out=out)

    wall, ms = timed_calls(call, steps, warmup)
    nbytes = step_bytes(N, n_tok, H, D)
    avg = float(np.mean(ms))
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"workload": f"{N} sequences x {n_tok} rows, H={H}, dk=dv={D}, bf16 q/k/v, fp32 state in place",
            "us_per_call": round(avg * 1e3, 2), "achieved_GBs": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "algorithmic_bytes": nbytes}


def cpu_baseline(inp, target_s=10.0):
    """Time the fp64 oracle on a bounded sample of the prefill workload: whole
    sequences, a subset of heads, sized from a pilot run to ~target_s."""
    import oracle
    from kda_inputs import to_f64
    threads = max(1, min(16, os.cpu_count() or 1))
    B, T, H, D = inp["q"].shape

    def run(nb, nh):
        sl = lambda t: to_f64(t[:nb, :, :nh])
        s0 = to_f64(inp["init_state"][:nb, :nh])
        args = (sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_g"]),
                to_f64(inp["beta"][:nb, :, :nh]))
        t0 = time.perf_counter()
        oracle.kda_forward(*args, init_state=s0, scale=inp["scale"], n_threads=threads)
        return time.perf_counter() - t0

    # pilot: one sequence, up to `threads` heads, one unit per thread
    t_pilot = run(1, min(H, threads))
    waves = max(1, int(target_s / max(t_pilot, 1e-3)))
    units = min(B * H, waves * threads)
    nh = H if units >= H else units
    nb = max(1, min(B, units // H))
    elapsed = run(nb, nh)
    token_heads = nb * T * nh
    return {"value": round(token_heads / elapsed / H, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{nb} x {T} tokens x {nh} of {H} heads ({token_heads} token-heads, fp64 token loop, "
                      f"{elapsed:.1f} s); tokens/s of the {H}-head mixer"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "step"], default="all",
                    help="restrict the run (profiling); the JSON line needs 'all'")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import gated_delta_rule_67_amd as kda

    res = {}
    if args.only in ("all", "prefill"):
        res["prefill"] = bench_prefill(kda, args.steps, args.warmup)
        print(f"prefill: mean {np.mean(res['prefill']['ms']) * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    if args.only in ("all", "step"):
        res["decode"] = bench_step(kda, "decode", args.steps, args.warmup)
        res["verify"] = bench_step(kda, "verify", args.steps, args.warmup)
        print(f"decode {res['decode']['us_per_call']} us, verify {res['verify']['us_per_call']} us",
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
        "dtype": os.environ.get("KDA_BENCH_DTYPE_LABEL", "bf16 in, f32 state"),
        "data": "synthetic (seeded; q,v~N(0,1), k L2-normalised, log_g=-softplus(N)*0.05, beta=sigmoid(N))",
        "config": {"workload": "chunked prefill, dense B=4 x T=4096, H=16, dk=dv=128, bf16 q/k/v, "
                               "fp32 log_g/beta/state, fp32 out, chunk 64",
                   "global_batch": 4, "seq_len": 4096, "heads": 16, "head_dim": 128},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "prefill_kernel_us": round(k_ms * 1e3, 2),
        "algorithmic_bytes_per_launch": p["bytes"],
        "mfma": {"achieved_TFLOPs": round(tflops, 2), "peak_TFLOPs": MFMA_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "algorithmic_flop_per_launch": p["flops"]},
        "decode": res["decode"],
        "verify": res["verify"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p["inp"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
