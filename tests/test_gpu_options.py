"""GPU parity of the call options: bf16 output and the in-kernel q / k L2
normalisation, through the C ABI, against the fp64 oracle.

bf16 out: the kernels round their fp32 result once to nearest even, so the
bf16 output must equal torch's rounding of the fp32 output of the same call
bit for bit (the fp32 arithmetic is the same; only the store differs), and
every element must lie within one bf16 rounding of the oracle plus the fp32
path's own bar: |gpu - oracle| <= 2^-8 |oracle| + tol * rms(oracle).

L2: the oracle normalises every q and k row by sqrt(sum of squares + 1e-6)
before the recurrence (oracle.qk_l2norm); the kernels must match that within
the usual bars on inputs that are not normalised (k ~ N(0, 1) scaled, q
scaled by 50, so that raw rows would leave the fp16 operand range).
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from gpu_helpers import TOL, err, oracle_full, oracle_threads, to_dev
from kda_inputs import to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_67_amd as kda  # noqa: E402

EPS = kda.QK_L2NORM_EPS


def bf16_bar(x, ref, tol):
    """max of |x - ref| / (2^-8 |ref| + tol rms(ref)): <= 1 passes."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(x))
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(x - ref) / (2.0 ** -8 * np.abs(ref) + tol * rms)))


def chunk(inp, **kw):
    d = to_dev(inp)
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_g"], d["beta"], init_state=d["init_state"],
                             cu_seqlens=d["cu_seqlens"], scale=inp["scale"], **kw)
    torch.cuda.synchronize()
    return out, fin


def unnormalised(inp, q_scale=50.0, k_scale=3.0, seed=0):
    """Replace k by raw N(0, 1) rows (not normalised) and scale q: inputs the
    in-kernel normalisation must handle."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal(inp["k"].shape).astype(np.float32) * k_scale
    q = inp["q"].float().numpy() * q_scale
    cast = (lambda a: torch.from_numpy(a).to(torch.bfloat16)) if inp["dtype"] == "bf16" else torch.from_numpy
    inp = dict(inp)
    inp["k"], inp["q"] = cast(k), cast(np.ascontiguousarray(q, dtype=np.float32))
    return inp


def oracle_l2(inp):
    cu = inp["cu_seqlens"].numpy().astype(np.int64) if inp["cu_seqlens"] is not None else None
    return oracle.kda_forward(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), to_f64(inp["log_g"]),
                              to_f64(inp["beta"]), init_state=to_f64(inp["init_state"]), cu_seqlens=cu,
                              scale=inp["scale"], n_threads=oracle_threads(), qk_l2norm_eps=EPS)


# ---------------------------------------------------------------- bf16 out
CASES = {
    "dense bf16 d128 ragged": dict(B=2, T=200, H=3, dk=128, dv=128, dtype="bf16", seed=301, init="normal",
                                   init_std=0.1),
    "packed bf16 d128 edges": dict(B=1, T=590, H=2, dk=128, dv=128, dtype="bf16", seed=302,
                                   lengths=[0, 1, 63, 64, 65, 0, 130, 7, 260], init="normal", init_std=0.1),
    "dense f32 d64 (recurrent)": dict(B=2, T=133, H=2, dk=64, dv=64, dtype="f32", seed=303),
    "dense bf16 d32 (recurrent)": dict(B=3, T=70, H=2, dk=32, dv=32, dtype="bf16", seed=304),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_fwd_bf16_out(name):
    inp = kda_inputs.make_inputs(**CASES[name])
    o32, f32 = chunk(inp)
    o16, f16 = chunk(inp, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    # one rounding of the same fp32 result, and the same final state
    assert torch.equal(o16, o32.to(torch.bfloat16)), name
    assert torch.equal(f16, f32)
    ref_o, _ = oracle_full(inp)
    bar = bf16_bar(o16.float().cpu().numpy(), ref_o, TOL[inp["dtype"]])
    print(f"[{name}] bf16 out: {bar:.3f} of the bar", flush=True)
    assert bar <= 1.0


def test_chunk_fwd_bf16_out_on_the_fallback_path():
    """Chunks on the exact per-token fallback store bf16 the same way."""
    inp = kda_inputs.make_inputs(B=2, T=64 * 3 + 9, H=2, dk=128, dv=128, dtype="bf16", seed=305,
                                 init="normal", init_std=0.05)
    g = inp["log_g"].numpy().copy()
    g[:, 70] = -np.inf
    g[:, 130:150, :, :8] = -3.0
    inp["log_g"] = torch.from_numpy(g)
    o32, _ = chunk(inp)
    o16, _ = chunk(inp, out_dtype=torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    ref_o, _ = oracle_full(inp)
    assert bf16_bar(o16.float().cpu().numpy(), ref_o, TOL["bf16"]) <= 1.0


def test_dense_prefill_workload_bf16_out():
    """The dense 4 x 4096-token, 16-head workload with bf16 out, whole tensor."""
    inp = kda_inputs.config("prefill")
    o16, fin = chunk(inp, out_dtype=torch.bfloat16)
    ref_o, ref_f = oracle_full(inp)
    bar = bf16_bar(o16.float().cpu().numpy(), ref_o, TOL["bf16"])
    e_f = err(fin.cpu().numpy(), ref_f)
    print(f"[prefill bf16 out] {bar:.3f} of the bar, err_final={e_f:.3e}", flush=True)
    assert bar <= 1.0 and e_f <= TOL["bf16"]


@pytest.mark.parametrize("n_tok", [1, 4])
def test_step_and_rows_bf16_out(n_tok):
    inp = kda_inputs.make_inputs(B=8, T=n_tok, H=4, dk=128, dv=128, dtype="bf16", seed=306 + n_tok)
    d = to_dev(inp)
    s32, s16 = d["init_state"].clone(), d["init_state"].clone()
    o32 = kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], s32)
    o16 = kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], s16, out_dtype=torch.bfloat16)
    r16, _ = kda.step_rows(d["q"], d["k"], d["v"], d["log_g"], d["beta"], d["init_state"],
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)
    assert torch.equal(r16, o16)
    ref_o, _ = oracle_full(inp)
    assert bf16_bar(o16.float().cpu().numpy(), ref_o, TOL["bf16"]) <= 1.0


# ---------------------------------------------------------------- L2 normalisation
L2_CASES = {
    "dense bf16 d128": dict(B=2, T=200, H=3, dk=128, dv=128, dtype="bf16", seed=311, init="normal",
                            init_std=0.1),
    "packed bf16 d128": dict(B=1, T=459, H=2, dk=128, dv=128, dtype="bf16", seed=312,
                             lengths=[0, 1, 63, 65, 200, 130], init="normal", init_std=0.1),
    "dense f32 d128 (recurrent)": dict(B=2, T=100, H=2, dk=128, dv=128, dtype="f32", seed=313),
    "dense bf16 d64 (recurrent)": dict(B=2, T=90, H=2, dk=64, dv=64, dtype="bf16", seed=314),
    "dense f32 d16 (recurrent)": dict(B=1, T=40, H=2, dk=16, dv=16, dtype="f32", seed=315),
}


@pytest.mark.parametrize("name", sorted(L2_CASES))
def test_chunk_fwd_qk_l2norm(name):
    inp = unnormalised(kda_inputs.make_inputs(**L2_CASES[name]), seed=316)
    out, fin = chunk(inp, qk_l2norm=True)
    ref_o, ref_f = oracle_l2(inp)
    e_o, e_f = err(out.cpu().numpy(), ref_o), err(fin.cpu().numpy(), ref_f)
    print(f"[L2 {name}] err_out={e_o:.3e} err_final={e_f:.3e}", flush=True)
    tol = TOL[inp["dtype"]]
    assert e_o <= tol and e_f <= tol
    # without the flag the same inputs give another result (the flag is not ignored);
    # unnormalised keys (|k|^2 ~ 1000) make the plain recurrence diverge, so
    # non-finite values are expected there
    plain, _ = chunk(inp)
    p = np.nan_to_num(plain.cpu().double().numpy(), nan=1e30, posinf=1e30, neginf=-1e30)
    assert np.abs(p - ref_o).max() > 10 * tol * np.sqrt(np.mean(ref_o ** 2))


def test_chunk_fwd_qk_l2norm_with_extreme_gates():
    """L2 normalisation on chunks that take the exact per-token fallback."""
    inp = unnormalised(kda_inputs.make_inputs(B=2, T=192, H=2, dk=128, dv=128, dtype="bf16", seed=317,
                                              init="normal", init_std=0.1), seed=318)
    rng = np.random.default_rng(319)
    g = -rng.uniform(0, 20, size=inp["log_g"].shape).astype(np.float32)
    g[:, 70] = -np.inf
    inp["log_g"] = torch.from_numpy(g)
    out, fin = chunk(inp, qk_l2norm=True)
    ref_o, ref_f = oracle_l2(inp)
    assert err(out.cpu().numpy(), ref_o) <= TOL["bf16"] and err(fin.cpu().numpy(), ref_f) <= TOL["bf16"]


@pytest.mark.parametrize("n_tok", [1, 4])
def test_step_rows_and_commit_qk_l2norm(n_tok):
    inp = unnormalised(kda_inputs.make_inputs(B=8, T=n_tok, H=4, dk=128, dv=128, dtype="bf16",
                                              seed=320 + n_tok), seed=322)
    d = to_dev(inp)
    st = d["init_state"].clone()
    out = kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], st, qk_l2norm=True)
    rows, deltas = kda.step_rows(d["q"], d["k"], d["v"], d["log_g"], d["beta"], d["init_state"], qk_l2norm=True)
    st2 = d["init_state"].clone()
    kda.step_commit(d["k"], d["log_g"], deltas, st2, torch.full((8,), n_tok, dtype=torch.int32, device="cuda"),
                    qk_l2norm=True)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_l2(inp)
    assert err(out.cpu().numpy(), ref_o) <= TOL["bf16"] and err(st.cpu().numpy(), ref_f) <= TOL["bf16"]
    assert torch.equal(rows, out)
    assert err(st2.cpu().numpy(), ref_f) <= TOL["bf16"]


def test_packed_workload_qk_l2norm_and_bf16_out():
    """The packed 65536-token, 32-head workload with both options, whole tensors:
    the raw k rows are scaled by 3 (not unit), so the normalisation matters."""
    inp = kda_inputs.config("varlen")
    inp = dict(inp, k=(inp["k"].float() * 3.0).to(torch.bfloat16))
    out, fin = chunk(inp, qk_l2norm=True, out_dtype=torch.bfloat16)
    ref_o, ref_f = oracle_l2(inp)
    bar = bf16_bar(out.float().cpu().numpy(), ref_o, TOL["bf16"])
    e_f = err(fin.cpu().numpy(), ref_f)
    print(f"[varlen L2 + bf16 out] {bar:.3f} of the bar, err_final={e_f:.3e}", flush=True)
    assert bar <= 1.0 and e_f <= TOL["bf16"]


# ---------------------------------------------------------------- KDA_VALIDATE=1
def test_validate_mode_passes_good_calls(monkeypatch):
    monkeypatch.setenv("KDA_VALIDATE", "1")
    inp = kda_inputs.make_inputs(B=1, T=300, H=2, dk=128, dv=128, dtype="bf16", seed=330,
                                 lengths=[0, 100, 200], init="normal", init_std=0.05)
    out, fin = chunk(inp)
    ref_o, ref_f = oracle_full(inp)
    assert err(out.cpu().numpy(), ref_o) <= TOL["bf16"] and err(fin.cpu().numpy(), ref_f) <= TOL["bf16"]
    d = to_dev(kda_inputs.make_inputs(B=4, T=2, H=2, dk=64, dv=64, dtype="f32", seed=331))
    kda.step(d["q"], d["k"], d["v"], d["log_g"], d["beta"], d["init_state"].clone(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()


def test_validate_mode_rejects_bad_device_inputs(monkeypatch):
    monkeypatch.setenv("KDA_VALIDATE", "1")
    inp = kda_inputs.make_inputs(B=1, T=300, H=2, dk=128, dv=128, dtype="bf16", seed=332,
                                 lengths=[100, 200], init="normal", init_std=0.05)
    d = to_dev(inp)
    call = lambda cu, g: kda.chunk_fwd(d["q"], d["k"], d["v"], g, d["beta"], init_state=d["init_state"],
                                       cu_seqlens=cu)
    for bad in ([0, 200, 100], [0, 100, 299], [5, 100, 300]):   # decreasing, short total, bad start
        with pytest.raises(kda.KdaError) as ei:
            call(torch.tensor(bad, dtype=torch.int32, device="cuda"), d["log_g"])
        assert ei.value.status == 2 and "KDA_VALIDATE" in str(ei.value)
    g = d["log_g"].clone()
    g[0, 150, 1, 3] = 0.5                                          # not a decay
    with pytest.raises(kda.KdaError) as ei:
        call(d["cu_seqlens"], g)
    assert ei.value.status == 2 and "positive" in str(ei.value)
    g[0, 150, 1, 3] = float("nan")
    with pytest.raises(kda.KdaError):
        call(d["cu_seqlens"], g)


def test_validate_mode_reports_non_finite_outputs(monkeypatch):
    """Unnormalised keys (|k|^2 ~ 1000) make the recurrence itself diverge: the
    call runs, and the mode reports the non-finite output."""
    monkeypatch.setenv("KDA_VALIDATE", "1")
    inp = unnormalised(kda_inputs.make_inputs(B=1, T=200, H=2, dk=128, dv=128, dtype="bf16", seed=333), seed=334)
    with pytest.raises(kda.KdaError) as ei:
        chunk(inp)
    assert ei.value.status == 7 and "not finite" in str(ei.value)



# ---------------------------------------------------------------- fused gated RMSNorm
def norm_inputs(inp, seed):
    rng = np.random.default_rng(seed)
    B, T, H, D = inp["v"].shape
    gate = torch.from_numpy(rng.standard_normal((B, T, H, D), dtype=np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal(D).astype(np.float32))
    return gate, w


def norm_bar(y, y_ref, o_ref, gate, w, eps, tol, bf16_out):
    """max |y - y_ref| / bar, per element, for y = norm(o): the prefill's own
    bar (|do| <= tol * rms of the whole output) carried through the norm.
    With r = sqrt(mean(o^2) + eps) of the row, d(o_i / r) = do_i / r -
    o_i dr / r^2 and |dr| <= max|do|, so |dy_i| <= |w_i sigmoid(g_i)| (1 +
    |o_i| / r) max|do| / r.  bf16 out adds two roundings of at most 2^-9 |y_i|
    each: o is stored in the output's dtype before the norm reads it back, and
    y is rounded once.  A row whose own RMS is far below the tensor's (a first
    token whose q.k nearly cancels) is amplified by the norm, and the bar grows
    with it."""
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y))
    do = tol * np.sqrt(np.mean(o_ref ** 2))
    r = np.sqrt(np.mean(o_ref ** 2, axis=-1, keepdims=True) + eps)
    gain = np.abs(to_f64(w)) / (1.0 + np.exp(-to_f64(gate)))
    bar = gain * (1.0 + np.abs(o_ref) / r) * do / r + 1e-6 * np.sqrt(np.mean(y_ref ** 2))
    if bf16_out:
        bar = bar + 2.0 ** -8 * np.abs(y_ref)
    return float(np.max(np.abs(y - y_ref) / bar))


def fused(inp, gate, w, eps, **kw):
    d = to_dev(inp)
    out, fin = kda.chunk_fwd_gated_norm(d["q"], d["k"], d["v"], d["log_g"], d["beta"], gate.cuda(), w.cuda(), eps,
                                        init_state=d["init_state"], cu_seqlens=d["cu_seqlens"], scale=inp["scale"],
                                        **kw)
    torch.cuda.synchronize()
    return out, fin


NORM_CASES = {
    "dense ragged": dict(B=2, T=200, H=3, dk=128, dv=128, dtype="bf16", seed=341, init="normal", init_std=0.1),
    "packed edges": dict(B=1, T=590, H=2, dk=128, dv=128, dtype="bf16", seed=342,
                         lengths=[0, 1, 63, 64, 65, 0, 130, 7, 260], init="normal", init_std=0.1),
}


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name", sorted(NORM_CASES))
def test_chunk_fwd_gated_norm(name, out_dtype):
    inp = kda_inputs.make_inputs(**NORM_CASES[name])
    gate, w = norm_inputs(inp, 343)
    out, fin = fused(inp, gate, w, 1e-6, out_dtype=out_dtype)
    ref_o, ref_f = oracle_full(inp)
    ref = oracle.gated_rmsnorm(ref_o, to_f64(gate), to_f64(w), 1e-6)
    bar = norm_bar(out.float().cpu().numpy(), ref, ref_o, gate, w, 1e-6, TOL["bf16"], out_dtype == torch.bfloat16)
    print(f"[norm {name} {out_dtype}] {bar:.3f} of the bar", flush=True)
    assert bar <= 1.0
    assert err(fin.cpu().numpy(), ref_f) <= TOL["bf16"]


def test_chunk_fwd_gated_norm_on_fallback_chunks():
    """Chunks on the exact per-token fallback (|beta| > 1 sends a chunk there)
    through the norm epilogue.  The trigger keeps every row's magnitude like the
    others': the norm rescales each row to unit RMS, so rows far below the
    tensor's RMS would turn the prefill's own rounding into large relative errors."""
    inp = kda_inputs.make_inputs(B=2, T=64 * 4 + 9, H=2, dk=128, dv=128, dtype="bf16", seed=344,
                                 init="normal", init_std=0.05)
    b = inp["beta"].numpy().copy()
    b[0, 70:72] = 1.5                           # chunk 1 of sequence 0
    b[1, 200] = -1.2                            # chunk 3 of sequence 1
    inp["beta"] = torch.from_numpy(b)
    gate, w = norm_inputs(inp, 345)
    out, _ = fused(inp, gate, w, 1e-5, out_dtype=torch.float32)
    ref_o, _ = oracle_full(inp)
    ref = oracle.gated_rmsnorm(ref_o, to_f64(gate), to_f64(w), 1e-5)
    assert norm_bar(out.cpu().numpy(), ref, ref_o, gate, w, 1e-5, TOL["bf16"], False) <= 1.0


def test_packed_workload_gated_norm_bf16_out():
    """The packed 65536-token, 32-head workload through the fused norm with bf16
    out (the mixer's output as the next projection takes it), whole tensor."""
    inp = kda_inputs.config("varlen")
    gate, w = norm_inputs(inp, 346)
    out, fin = fused(inp, gate, w, 1e-6)
    ref_o, ref_f = oracle_full(inp)
    ref = oracle.gated_rmsnorm(ref_o, to_f64(gate), to_f64(w), 1e-6)
    bar = norm_bar(out.float().cpu().numpy(), ref, ref_o, gate, w, 1e-6, TOL["bf16"], True)
    e_f = err(fin.cpu().numpy(), ref_f)
    print(f"[varlen fused norm bf16 out] {bar:.3f} of the bar, err_final={e_f:.3e}", flush=True)
    assert bar <= 1.0 and e_f <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128)])
def test_gated_norm_on_the_recurrent_path(dtype, d):
    """Configurations outside the chunked MFMA path (d < 128, fp32 q/k/v) take
    the token-recurrent prefill, then the same in-place norm."""
    inp = kda_inputs.make_inputs(B=2, T=75, H=2, dk=d, dv=d, dtype=dtype, seed=347, init="normal", init_std=0.1)
    B, T, H, D = inp["v"].shape
    rng = np.random.default_rng(348)
    g32 = rng.standard_normal((B, T, H, D), dtype=np.float32)
    gate = torch.from_numpy(g32).to(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(g32)
    w = torch.from_numpy(rng.standard_normal(D).astype(np.float32))
    out, fin = fused(inp, gate, w, 1e-6, out_dtype=torch.float32)
    ref_o, ref_f = oracle_full(inp)
    ref = oracle.gated_rmsnorm(ref_o, to_f64(gate), to_f64(w), 1e-6)
    tol = TOL["bf16"] if dtype == "bf16" else TOL["f32"]
    bar = norm_bar(out.cpu().numpy(), ref, ref_o, gate, w, 1e-6, tol, False)
    print(f"[norm recurrent {dtype} d={d}] {bar:.3f} of the bar", flush=True)
    assert bar <= 1.0
    assert err(fin.cpu().numpy(), ref_f) <= tol
