"""GPU parity of speculative verify: kda_step_rows then kda_step_commit.

Rows t = 0 .. n_tok-1 are scored without touching the state; each sequence
then keeps its first accept[n] rows.  The reference for a sequence that keeps
m rows is the fp64 oracle run on its first m rows alone (verify row t uses
slot t; rejected rows leave no trace).  Tolerances as in the other parity
tests.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from gpu_helpers import TOL, err, oracle_threads, to_dev
from kda_inputs import to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_67_amd as kda  # noqa: E402


def oracle_prefix(inp, m):
    """Oracle on the first m rows of every sequence: (out [N,m,H,dv], final)."""
    if m == 0:
        return None, inp["init_state"].double().numpy()
    cut = lambda t: to_f64(t[:, :m])
    return oracle.kda_forward(cut(inp["q"]), cut(inp["k"]), cut(inp["v"]), cut(inp["log_g"]),
                              cut(inp["beta"]), init_state=to_f64(inp["init_state"]), scale=inp["scale"],
                              n_threads=oracle_threads())


def run_rows(d, inp, state):
    return kda.step_rows(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, scale=inp["scale"])


@pytest.mark.parametrize("dtype,d,n_tok", [("bf16", 128, 4), ("f32", 64, 3), ("bf16", 16, 5)])
def test_rows_match_step_and_keep_the_state(dtype, d, n_tok):
    inp = kda_inputs.make_inputs(B=6, T=n_tok, H=3, dk=d, dv=d, dtype=dtype, seed=40 + d,
                                 init="normal", init_std=0.05)
    dv = to_dev(inp)
    s_rows = dv["init_state"].clone()
    out_rows, deltas = run_rows(dv, inp, s_rows)
    s_step = dv["init_state"].clone()
    out_step = kda.step(dv["q"], dv["k"], dv["v"], dv["log_g"], dv["beta"], s_step, scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(s_rows, dv["init_state"])          # the rows pass reads the state only
    assert torch.equal(out_rows, out_step)                 # same kernel, same outputs
    ref_o, _ = oracle_prefix(inp, n_tok)
    assert err(out_rows.cpu().numpy(), ref_o) <= TOL[dtype]
    # committing every row is kda_step's state update
    accept = torch.full((6,), n_tok, dtype=torch.int32, device="cuda")
    kda.step_commit(dv["k"], dv["log_g"], deltas, s_rows, accept)
    torch.cuda.synchronize()
    e_same = err(s_rows.cpu().numpy(), s_step.cpu().numpy())
    print(f"[rows {dtype} d={d} n_tok={n_tok}] commit vs step {e_same:.2e}", flush=True)
    assert e_same <= 1e-6


def test_commit_keeps_each_sequences_accepted_prefix():
    """Every accept count from 0 to n_tok, plus out-of-range values (clamped)."""
    n_tok, N = 4, 8
    inp = kda_inputs.make_inputs(B=N, T=n_tok, H=4, dk=128, dv=128, dtype="bf16", seed=50,
                                 init="normal", init_std=0.05)
    dv = to_dev(inp)
    state = dv["init_state"].clone()
    _, deltas = run_rows(dv, inp, state)
    acc = [0, 1, 2, 3, 4, -3, 99, 2]
    kda.step_commit(dv["k"], dv["log_g"], deltas, state, torch.tensor(acc, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got = state.cpu()
    for m in sorted(set(min(max(a, 0), n_tok) for a in acc)):
        seqs = [i for i, a in enumerate(acc) if min(max(a, 0), n_tok) == m]
        _, ref_f = oracle_prefix(inp, m)
        e = err(got[seqs].numpy(), ref_f[seqs])
        print(f"[commit m={m} seqs={seqs}] err={e:.2e}", flush=True)
        if m == 0:
            assert torch.equal(got[seqs], inp["init_state"][seqs])
        else:
            assert e <= TOL["bf16"]


def test_verify_workload_with_random_acceptance():
    """The 64 x 4-row, 32-head verify workload; each sequence keeps a random prefix."""
    inp = kda_inputs.config("verify")
    N, n_tok = inp["q"].shape[:2]
    dv = to_dev(inp)
    state = dv["init_state"].clone()
    out, deltas = run_rows(dv, inp, state)
    acc = np.random.default_rng(7).integers(0, n_tok + 1, size=N).astype(np.int32)
    kda.step_commit(dv["k"], dv["log_g"], deltas, state, torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    ref_o, _ = oracle_prefix(inp, n_tok)
    assert err(out.cpu().numpy(), ref_o) <= TOL["bf16"]
    got = state.cpu()
    worst = 0.0
    for m in range(n_tok + 1):
        seqs = np.nonzero(acc == m)[0].tolist()
        if not seqs:
            continue
        _, ref_f = oracle_prefix(inp, m)
        worst = max(worst, err(got[seqs].numpy(), ref_f[seqs]))
    print(f"[verify workload, random acceptance] worst state err {worst:.2e}", flush=True)
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("dtype,rows", [("bf16", 8), ("f32", 5)])
def test_prompt_tail_through_multi_row_steps(dtype, rows):
    """A 205-token prompt: its three whole 64-token chunks through
    kda_chunk_fwd, the 13-token tail through kda_step calls of `rows` rows
    (the batched sub-chunk walk); and the whole prompt through that walk
    alone.  Both equal the oracle on the whole prompt."""
    T, done = 205, 192
    inp = kda_inputs.make_inputs(B=3, T=T, H=4, dk=128, dv=128, dtype=dtype, seed=90 + rows,
                                 init="normal", init_std=0.05)
    dv = to_dev(inp)
    sl = lambda x, a, b: x[:, a:b].contiguous()

    def walk(state, start):
        outs = []
        for a in range(start, T, rows):
            b = min(a + rows, T)
            outs.append(kda.step(sl(dv["q"], a, b), sl(dv["k"], a, b), sl(dv["v"], a, b), sl(dv["log_g"], a, b),
                                 sl(dv["beta"], a, b), state, scale=inp["scale"]))
        return outs

    o_head, state = kda.chunk_fwd(sl(dv["q"], 0, done), sl(dv["k"], 0, done), sl(dv["v"], 0, done),
                                  sl(dv["log_g"], 0, done), sl(dv["beta"], 0, done), init_state=dv["init_state"],
                                  scale=inp["scale"])
    o_mixed = torch.cat([o_head] + walk(state, done), 1)
    s_walk = dv["init_state"].clone()
    o_walk = torch.cat(walk(s_walk, 0), 1)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_prefix(inp, T)
    for name, o, f in (("chunks + tail", o_mixed, state), ("sub-chunk walk", o_walk, s_walk)):
        eo, ef = err(o.cpu().numpy(), ref_o), err(f.cpu().numpy(), ref_f)
        print(f"[prompt {dtype} rows={rows} {name}] out {eo:.2e} state {ef:.2e}", flush=True)
        assert eo <= TOL[dtype] and ef <= TOL[dtype]
