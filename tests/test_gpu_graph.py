"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

Each call is warmed up eagerly once (the first call on a device sets kernel
attributes), then captured and replayed several times with eager work and
synchronisations in between; every replay must give the eager results bit
for bit.  No kernel here records a memset, and every output is written in
full by the kernels, so replays are exact.
"""
import pytest
import torch

import kda_inputs
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_67_amd as kda  # noqa: E402


def replay_matches(fn, outputs_of, n_replays=3):
    """fn() enqueues work on the current stream and returns its outputs."""
    eager = [t.clone() for t in outputs_of(fn())]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    for i in range(n_replays):
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        for t in outputs_of(res):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs_of(res), eager):
            assert torch.equal(a, b), f"replay {i} differs"
        del junk


def test_prefill_and_decode_in_a_graph():
    inp = kda_inputs.make_inputs(B=2, T=300, H=4, dk=128, dv=128, dtype="bf16", seed=500)
    d = to_dev(inp)
    st_src = d["init_state"].clone()
    step_in = kda_inputs.make_inputs(B=2, T=1, H=4, dk=128, dv=128, dtype="bf16", seed=501)
    ds = to_dev(step_in)
    state = torch.empty_like(st_src)

    def fn():
        out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"])
        state.copy_(fin)
        o1 = kda.step(ds["q"], ds["k"], ds["v"], ds["log_g"], ds["beta"], state)
        return out, fin, o1, state

    replay_matches(fn, lambda res: res)


def test_backward_conv_and_norm_in_a_graph():
    inp = kda_inputs.make_inputs(B=1, T=200, H=2, dk=64, dv=64, dtype="f32", seed=510,
                                 lengths=[70, 0, 130], init="normal")
    up = kda_inputs.upstream_grads(inp, seed=511)
    d = to_dev(inp)
    do, dfin = up["d_out"].cuda(), up["d_final"].cuda()
    ci = kda_inputs.conv_inputs(B=2, T=100, channels=256, K=4, dtype="bf16", seed=512)
    x, w, c0 = ci["x"].cuda(), ci["weight"].cuda(), ci["init_cache"].cuda()
    o = torch.randn((2, 33, 4, 64), device="cuda")
    gt = torch.randn((2, 33, 4, 64), device="cuda").to(torch.bfloat16)
    wn = torch.randn(64, device="cuda")

    def fn():
        g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], do, init_state=d["init_state"],
                          cu_seqlens=d["cu_seqlens"], d_final=dfin)
        y, fin = kda.short_conv(x, w, init_cache=c0, activation=1)
        yn = kda.gated_rmsnorm(o, gt, wn, 1e-6)
        return [g[n] for n in ("dq", "dk", "dv", "dlog_g", "dbeta", "d_init_state")] + [y, fin, yn]

    replay_matches(fn, lambda res: res)
