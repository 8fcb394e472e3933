"""GPU parity: libkda (through its C ABI) against the fp64 oracle.

Both sides receive the same seeded inputs (kda_inputs).  The metric is
max |gpu - oracle| / rms(oracle) per tensor, against 1e-4 for fp32 q/k/v and
2e-2 for bf16 q/k/v; final states meet the same bound.  Full-size workloads
run in the launch configuration the benchmark times, and every one of them
(the 65536-token packed workload included) is compared with the oracle
element by element over the whole output and final-state tensors.
"""
import numpy as np
import pytest
import torch

import kda_inputs
from gpu_helpers import TOL, err, oracle_full, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_67_amd as kda  # noqa: E402

# The chunked path's serial pass has two forms: four 32-column workgroups per
# (sequence or document, head) of eight waves ("tile8") or of four waves, two
# per CU ("tile4").  Every test runs under both (the switch only affects bf16
# d = 128 prefill).
SCAN_FORMS = ["tile8", "tile4"]


@pytest.fixture(params=SCAN_FORMS, autouse=True)
def scan_form(request, monkeypatch):
    monkeypatch.setenv("KDA_PREFILL_PATH", request.param)
    return request.param

def run_chunk(inp, **kw):
    d = to_dev(inp)
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"],
                             cu_seqlens=d["cu_seqlens"], scale=inp["scale"], **kw)
    torch.cuda.synchronize()
    return out, fin


def check_full(inp, tag):
    out, fin = run_chunk(inp)
    ref_o, ref_f = oracle_full(inp)
    e_o, e_f = err(out.cpu().numpy(), ref_o), err(fin.cpu().numpy(), ref_f)
    print(f"[{tag}] err_out={e_o:.3e} err_final={e_f:.3e}", flush=True)
    tol = TOL[inp["dtype"]]
    assert e_o <= tol and e_f <= tol, (tag, e_o, e_f)
    return e_o, e_f


# ---------------------------------------------------------------- the five workloads
def test_tiny_fp32_workload():
    inp = kda_inputs.config("tiny")
    assert inp["scale"] == 0.25
    check_full(inp, "tiny")


def test_dense_prefill_workload():
    inp = kda_inputs.config("prefill")
    check_full(inp, "prefill B4 T4096 H16")


def test_packed_varlen_workload():
    """The packed 65536-token, 32-head workload (26 documents, log-uniform
    lengths 64..16384, zero initial states): the whole output [1, 65536, 32,
    128] and the whole final state [26, 32, 128, 128] against the oracle."""
    inp = kda_inputs.config("varlen")
    lens = np.diff(inp["cu_seqlens"].numpy())
    print(f"[varlen] {len(lens)} documents, longest {lens.max()}, shortest {lens.min()}", flush=True)
    check_full(inp, "packed varlen 65536 tokens H32")


@pytest.mark.parametrize("name", ["decode", "verify"])
def test_step_workloads(name):
    inp = kda_inputs.config(name)
    d = to_dev(inp)
    state = d["init_state"].clone()
    out = kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], state, scale=inp["scale"])
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_full(inp)
    e_o, e_f = err(out.cpu().numpy(), ref_o), err(state.cpu().numpy(), ref_f)
    print(f"[{name}] err_out={e_o:.3e} err_state={e_f:.3e}", flush=True)
    assert e_o <= TOL["bf16"] and e_f <= TOL["bf16"]


# ---------------------------------------------------------------- shapes and edge cases
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_dense_ragged_all_dims(dtype, d):
    """Several chunks plus a ragged tail (200 = 3*64 + 8 tokens)."""
    inp = kda_inputs.make_inputs(B=2, T=200, H=3, dk=d, dv=d, dtype=dtype, seed=10 + d,
                                 gate_scale=0.1, init="normal", init_std=0.1)
    check_full(inp, f"dense {dtype} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_edge_lengths(dtype):
    """Empty, single-token, exactly-one-chunk, one-past and multi-chunk documents."""
    lens = [0, 1, 63, 64, 65, 0, 130, 7, 257]
    inp = kda_inputs.make_inputs(B=1, T=sum(lens), H=4, dk=128, dv=128, dtype=dtype, seed=20,
                                 lengths=lens, init="normal", init_std=0.1)
    out, fin = check_full(inp, f"packed edges {dtype}")
    _, fin_dev = run_chunk(inp)
    # an empty document's final state is its initial state
    s0 = inp["init_state"]
    assert torch.equal(fin_dev[0].cpu(), s0[0]) and torch.equal(fin_dev[5].cpu(), s0[5])


def test_long_single_document():
    """One document of 257 chunks with a ragged tail: the scan's long serial walk."""
    lens = [256 * 64 + 37]
    inp = kda_inputs.make_inputs(B=1, T=sum(lens), H=2, dk=128, dv=128, dtype="bf16", seed=22,
                                 lengths=lens, init="normal", init_std=0.05)
    check_full(inp, "packed one long document")


@pytest.mark.parametrize("n_docs", [5000, 17000])
def test_many_documents(n_docs):
    """Thousands of short documents (0 to 40 tokens): the longest-first sort
    covers up to 16384 documents (a bitonic network over the next power of
    two), problems with more are scanned in their given order, and the chunk
    map walks the documents in several blocks of 1024."""
    rng = np.random.default_rng(23)
    lens = [int(x) for x in rng.integers(0, 41, size=n_docs)]
    lens[0], lens[1] = 0, 1
    inp = kda_inputs.make_inputs(B=1, T=sum(lens), H=2, dk=128, dv=128, dtype="bf16", seed=24,
                                 lengths=lens, init="normal", init_std=0.05)
    check_full(inp, f"packed {n_docs} short documents")


def test_packed_zero_initial_state():
    lens = [100, 28, 256, 1]
    inp = kda_inputs.make_inputs(B=1, T=sum(lens), H=2, dk=128, dv=128, dtype="bf16", seed=21,
                                 lengths=lens, init="zeros")
    check_full(inp, "packed zero init")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_gates(dtype):
    """Strong decays: log_g uniform in [-20, 0] with some -inf (full reset) tokens."""
    inp = kda_inputs.make_inputs(B=2, T=192, H=2, dk=128, dv=128, dtype=dtype, seed=30,
                                 init="normal", init_std=0.1)
    rng = np.random.default_rng(31)
    g = -rng.uniform(0, 20, size=inp["log_g"].shape).astype(np.float32)
    g[:, 70] = -np.inf                         # every channel wiped at token 70
    g[0, 5:9, 1, :64] = -np.inf                # half the channels of one head
    inp["log_g"] = torch.from_numpy(g)
    check_full(inp, f"extreme gates {dtype}")


def test_identity_tokens_keep_state_exactly():
    """beta = 0 and log_g = 0: the final state equals the initial state bit for bit."""
    inp = kda_inputs.make_inputs(B=2, T=130, H=2, dk=128, dv=128, dtype="bf16", seed=40)
    inp["beta"] = torch.zeros_like(inp["beta"])
    inp["log_g"] = torch.zeros_like(inp["log_g"])
    out, fin = run_chunk(inp)
    assert torch.equal(fin.cpu(), inp["init_state"])
    ref_o, _ = oracle_full(inp)
    assert err(out.cpu().numpy(), ref_o) <= TOL["bf16"]


def test_resume_in_place_matches_one_run():
    """Run [0, t) then [t, T) from the first call's final state, written in place
    over the initial state (init_state aliases final_state)."""
    inp = kda_inputs.make_inputs(B=2, T=300, H=4, dk=128, dv=128, dtype="bf16", seed=50)
    d = to_dev(inp)
    full_o, full_f = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"])
    t = 100
    st = d["init_state"].clone()
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o1, _ = kda.chunk_fwd(*(sl(d[n], 0, t) for n in ("q", "k", "v", "log_g", "beta")), init_state=st,
                          final_state=st)
    o2, _ = kda.chunk_fwd(*(sl(d[n], t, 300) for n in ("q", "k", "v", "log_g", "beta")), init_state=st,
                          final_state=st)
    torch.cuda.synchronize()
    ref = full_o.cpu().numpy()
    assert err(torch.cat([o1, o2], 1).cpu().numpy(), ref) <= 2e-2
    assert err(st.cpu().numpy(), full_f.cpu().numpy()) <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_rows_equal_single_steps_and_prefill(dtype):
    """n_tok = 64 verify == 64 single-token decodes == prefill from that state."""
    inp = kda_inputs.make_inputs(B=3, T=64, H=2, dk=128, dv=128, dtype=dtype, seed=60,
                                 init="normal", init_std=0.1)
    d = to_dev(inp)
    s_multi = d["init_state"].clone()
    o_multi = kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], s_multi)
    s_one = d["init_state"].clone()
    outs = []
    for t in range(64):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(kda.step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["log_g"]), sl(d["beta"]), s_one))
    o_pre, f_pre = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"])
    torch.cuda.synchronize()
    o_one = torch.cat(outs, 1)
    assert torch.allclose(o_multi, o_one, rtol=1e-5, atol=1e-5)
    assert torch.allclose(s_multi, s_one, rtol=1e-5, atol=1e-5)
    ref_o, ref_f = oracle_full(inp)
    tol = TOL[dtype]
    for o, f in ((o_multi, s_multi), (o_pre, f_pre)):
        assert err(o.cpu().numpy(), ref_o) <= tol and err(f.cpu().numpy(), ref_f) <= tol


def test_runs_on_a_side_stream():
    inp = kda_inputs.make_inputs(B=1, T=128, H=2, dk=64, dv=64, dtype="bf16", seed=70)
    d = to_dev(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"])
    s.synchronize()
    ref_o, ref_f = oracle_full(inp)
    assert err(out.cpu().numpy(), ref_o) <= 2e-2 and err(fin.cpu().numpy(), ref_f) <= 2e-2


def test_final_state_optional():
    inp = kda_inputs.make_inputs(B=1, T=70, H=2, dk=32, dv=32, dtype="f32", seed=80)
    out, fin = run_chunk(inp, final_state=False)
    assert fin is None
    ref_o, _ = oracle_full(inp)
    assert err(out.cpu().numpy(), ref_o) <= 1e-4


def test_mixed_fast_and_fallback_chunks():
    """One sequence whose chunks alternate between the MFMA path and the exact
    token-by-token fallback (strong decays, a full reset, large values)."""
    T = 64 * 6 + 17
    inp = kda_inputs.make_inputs(B=2, T=T, H=4, dk=128, dv=128, dtype="bf16", seed=90,
                                 init="normal", init_std=0.05)
    g = inp["log_g"].numpy().copy()
    g[:, 64 + 10] = -np.inf                    # chunk 1: full reset at one token
    g[:, 192:256, :, :16] = -2.5               # chunk 3: strong decay on 16 channels
    g[1, 320:330, 2] = -7.0                    # chunk 5, one sequence/head only
    inp["log_g"] = torch.from_numpy(g)
    v = inp["v"].float().numpy().copy()
    v[0, 260:262] *= 3e4                       # chunk 4: values beyond the fp16 operand bound
    inp["v"] = torch.from_numpy(v).to(torch.bfloat16)
    check_full(inp, "mixed fast/fallback chunks")


def test_mfma_path_matches_recurrent_path(monkeypatch, scan_form):
    """The chunked kernel agrees with the token-recurrent one (and with the oracle)."""
    inp = kda_inputs.make_inputs(B=2, T=333, H=4, dk=128, dv=128, dtype="bf16", seed=91)
    out_c, fin_c = run_chunk(inp)
    monkeypatch.setenv("KDA_PREFILL_PATH", "recurrent")
    out_r, fin_r = run_chunk(inp)
    monkeypatch.setenv("KDA_PREFILL_PATH", scan_form)
    ref_o, ref_f = oracle_full(inp)
    e_c = err(out_c.cpu().numpy(), ref_o)
    e_r = err(out_r.cpu().numpy(), ref_o)
    print(f"[paths] chunk err={e_c:.3e} recurrent err={e_r:.3e}", flush=True)
    assert e_r <= 1e-4                          # fp32 token loop
    assert e_c <= TOL["bf16"]
    assert err(out_c.cpu().numpy(), out_r.cpu().numpy()) <= TOL["bf16"]
    assert err(fin_c.cpu().numpy(), fin_r.cpu().numpy()) <= TOL["bf16"]


def test_workspace_reused_and_contents_ignored():
    """A caller workspace serves calls of different shapes, and whatever it
    holds on entry (here NaN bytes) does not leak into the results."""
    big = kda_inputs.make_inputs(B=1, T=700, H=3, dk=128, dv=128, dtype="bf16", seed=92,
                                 lengths=[300, 0, 64, 336], init="normal", init_std=0.05)
    small = kda_inputs.make_inputs(B=2, T=129, H=3, dk=128, dv=128, dtype="bf16", seed=93)
    need = max(kda.workspace_bytes(4, 700, 3, 128, packed=True), kda.workspace_bytes(2, 129, 3, 128, packed=False))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for inp, tag in ((big, "ws packed"), (small, "ws dense"), (big, "ws packed again")):
        out, fin = run_chunk(inp, workspace=ws)
        ref_o, ref_f = oracle_full(inp)
        e_o, e_f = err(out.cpu().numpy(), ref_o), err(fin.cpu().numpy(), ref_f)
        print(f"[{tag}] err_out={e_o:.3e} err_final={e_f:.3e}", flush=True)
        assert e_o <= TOL["bf16"] and e_f <= TOL["bf16"]


SLOT_BYTES, FLAG_OFF = 74752, 74240  # workspace slot of one (chunk, head); its eight per-wave fallback bytes


@pytest.mark.parametrize("gates", ["gate_scale 1.0", "uniform -5..0", "uniform -20..0 with resets"])
def test_strong_gates_stay_on_the_mfma_path(gates):
    """Gates far stronger than the workloads' 0.05 scale: every chunk must still
    take the MFMA path (its diagonal tiles from the pair tree; no prep
    fallback flag set) and match the oracle."""
    B, T, H = 2, 640, 4
    over = {"gate_scale 1.0": dict(gate_scale=1.0), "uniform -5..0": dict(gate_uniform=5.0),
            "uniform -20..0 with resets": dict(gate_uniform=20.0)}[gates]
    inp = kda_inputs.make_inputs(B=B, T=T, H=H, dk=128, dv=128, dtype="bf16", seed=95, init="normal",
                                 init_std=0.05, **over)
    if "resets" in gates:
        g = inp["log_g"].numpy().copy()
        g[:, 70] = -np.inf
        g[0, 300:305, 1, :40] = -np.inf
        inp["log_g"] = torch.from_numpy(g)
    ws = torch.empty(kda.workspace_bytes(B, T, H, 128, packed=False), dtype=torch.uint8, device="cuda")
    out, fin = run_chunk(inp, workspace=ws)
    n_slots = B * (T // 64) * H
    flags = ws[: n_slots * SLOT_BYTES].view(n_slots, SLOT_BYTES)[:, FLAG_OFF:FLAG_OFF + 8]
    frac = float((flags != 0).any(dim=1).float().mean())
    ref_o, ref_f = oracle_full(inp)
    e_o, e_f = err(out.cpu().numpy(), ref_o), err(fin.cpu().numpy(), ref_f)
    print(f"[strong gates {gates}] fallback fraction {frac:.3f} err_out={e_o:.3e} err_final={e_f:.3e}", flush=True)
    assert frac == 0.0
    assert e_o <= TOL["bf16"] and e_f <= TOL["bf16"]


def test_scan_forms_agree(monkeypatch):
    """The two forms of the serial pass give the same results on a packed batch."""
    inp = kda_inputs.make_inputs(B=1, T=1500, H=4, dk=128, dv=128, dtype="bf16", seed=96,
                                 lengths=[1, 700, 63, 0, 736], init="normal", init_std=0.05)
    res = {}
    for form in SCAN_FORMS:
        monkeypatch.setenv("KDA_PREFILL_PATH", form)
        res[form] = run_chunk(inp)
    o1, f1 = res["tile8"]
    for form in SCAN_FORMS[1:]:
        o2, f2 = res[form]
        e_o, e_f = err(o2.cpu().numpy(), o1.cpu().numpy()), err(f2.cpu().numpy(), f1.cpu().numpy())
        print(f"[tile8 vs {form}] out={e_o:.3e} final={e_f:.3e}", flush=True)
        assert e_o <= 1e-5 and e_f <= 1e-5
