"""Pins of the oracle's reverse mode (CPU only).

The backward of the KDA recurrence is the gradient of the scalar loss
L = sum(d_out * out) + sum(d_final * final_state) with respect to every input
(NeMo glm5_next.layers documents ``_torch_recurrent_kda`` as the differentiable
reference; training is what the backward is for).  Nothing here re-types the
oracle's reverse loop:

* central finite differences of the (separately pinned) forward oracle, for
  every element of every input, on small problems, including beta outside
  [0, 1] and strong decays;
* a closed form when nothing is written (beta = 0) and nothing decays (g = 0);
* exact separation at a log_g = -inf gate (no gradient flows back through a
  token that erases the state);
* packed documents equal separate problems, dense equals packed, and the
  gradients are linear in (d_out, d_final).

``KDA_ORACLE_LIB`` may name another compiled oracle library; the mutation test
uses it to show that planted mistakes in the reverse mode fail these pins.
"""
import os

import numpy as np
import pytest

import oracle

_LIB = oracle.load(os.environ["KDA_ORACLE_LIB"]) if os.environ.get("KDA_ORACLE_LIB") else None
NAMES = ("q", "k", "v", "log_g", "beta", "init_state")
GRAD = {"q": "dq", "k": "dk", "v": "dv", "log_g": "dlog_g", "beta": "dbeta", "init_state": "d_init_state"}


def fwd(x, **kw):
    return oracle.kda_forward(x["q"], x["k"], x["v"], x["log_g"], x["beta"], init_state=x["init_state"],
                              lib=_LIB, **kw)


def bwd(x, d_out, d_final, **kw):
    return oracle.kda_backward(x["q"], x["k"], x["v"], x["log_g"], x["beta"], init_state=x["init_state"],
                               d_out=d_out, d_final=d_final, lib=_LIB, **kw)


def problem(rng, B, T, H, dk, dv, N=None, gate=0.5):
    N = B if N is None else N
    x = {"q": rng.standard_normal((B, T, H, dk)),
         "k": rng.standard_normal((B, T, H, dk)) * 0.7,
         "v": rng.standard_normal((B, T, H, dv)),
         "log_g": -np.logaddexp(0, rng.standard_normal((B, T, H, dk))) * gate,
         "beta": rng.uniform(-0.5, 1.7, (B, T, H)),          # beta outside [0, 1] too
         "init_state": rng.standard_normal((N, H, dk, dv)) * 0.5}
    d_out = rng.standard_normal((B, T, H, dv))
    d_final = rng.standard_normal((N, H, dk, dv))
    return x, d_out, d_final


def loss(x, d_out, d_final, **kw):
    out, fin = fwd(x, **kw)
    return float(np.sum(out * d_out) + np.sum(fin * d_final))


def finite_differences(x, d_out, d_final, h=1e-6, **kw):
    fd = {}
    for name in NAMES:
        g = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            g[idx] = (loss(xp, d_out, d_final, **kw) - loss(xm, d_out, d_final, **kw)) / (2 * h)
        fd[name] = g
    return fd


def assert_grads_close(got, ref, tol):
    for name in NAMES:
        a, b = got[GRAD[name]], ref[name]
        scale = max(1.0, np.abs(b).max())
        assert np.abs(a - b).max() <= tol * scale, (name, np.abs(a - b).max(), scale)


# --------------------------------------------------------------------------- finite differences
@pytest.mark.parametrize("B,T,H,dk,dv,gate,seed", [(2, 5, 2, 3, 2, 0.5, 1), (1, 7, 1, 2, 4, 4.0, 2),
                                                   (1, 4, 1, 4, 3, 0.05, 3)])
def test_B1_finite_differences_dense(B, T, H, dk, dv, gate, seed):
    rng = np.random.default_rng(seed)
    x, d_out, d_final = problem(rng, B, T, H, dk, dv, gate=gate)
    kw = {"scale": 0.7}
    g = bwd(x, d_out, d_final, **kw)
    assert_grads_close(g, finite_differences(x, d_out, d_final, **kw), 1e-7)


def test_B1_finite_differences_packed():
    """Three documents (one empty) in one packed row, each from its own state."""
    rng = np.random.default_rng(11)
    lens = [3, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x, d_out, d_final = problem(rng, 1, sum(lens), 2, 3, 2, N=len(lens))
    kw = {"scale": 0.9, "cu_seqlens": cu}
    g = bwd(x, d_out, d_final, **kw)
    fd = finite_differences(x, d_out, d_final, **kw)
    assert_grads_close(g, fd, 1e-7)
    # the empty document passes its final-state gradient straight to its initial state
    np.testing.assert_array_equal(g["d_init_state"][1], d_final[1])


def test_B1_default_scale_is_inverse_sqrt_dk():
    rng = np.random.default_rng(12)
    x, d_out, d_final = problem(rng, 1, 3, 1, 4, 2)
    a = bwd(x, d_out, d_final)
    b = bwd(x, d_out, d_final, scale=0.5)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


# --------------------------------------------------------------------------- closed form
def test_B2_no_write_no_decay_closed_form():
    """beta = 0 and g = 0: the state stays S0, o_t = scale S0^T q_t.  Then
    dq_t = scale S0 do_t; dv = dk = dlog_g's write terms vanish except through
    the read-back; dL/dS_t = d_final + scale sum_{u>t} q_u do_u^T, so
    dbeta_t = (dL/dS_t^T k_t) . (v_t - S0^T k_t) and
    dlog_g_t[i] = sum_j dL/dS_t[i,j] S0[i,j] (with dL/dS_t taken after token t's
    own output term), d_init = d_final + scale sum_t q_t do_t^T."""
    rng = np.random.default_rng(21)
    T, dk, dv, scale = 6, 4, 3, 0.8
    x, d_out, d_final = problem(rng, 1, T, 1, dk, dv)
    x["beta"][:] = 0.0
    x["log_g"][:] = 0.0
    g = bwd(x, d_out, d_final, scale=scale)
    S0 = x["init_state"][0, 0]
    q, k, v, do = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], d_out[0, :, 0]
    dS = d_final[0, 0].copy()
    for t in range(T - 1, -1, -1):
        dS = dS + scale * np.outer(q[t], do[t])       # dL/dS_t, output term of token t included
        np.testing.assert_allclose(g["dq"][0, t, 0], scale * S0 @ do[t], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g["dbeta"][0, t, 0], (dS.T @ k[t]) @ (v[t] - S0.T @ k[t]), rtol=1e-12,
                                   atol=1e-12)
        np.testing.assert_allclose(g["dlog_g"][0, t, 0], np.sum(dS * S0, axis=1), rtol=1e-12, atol=1e-12)
    assert np.all(g["dv"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["d_init_state"][0, 0], dS, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- invariants
def test_B3_erasing_gate_separates_the_gradients():
    """log_g = -inf on every channel of token r erases the state: the gradients
    of tokens before r are those of the prefix alone with no final-state
    gradient, and those from r on are those of the suffix run from a zero
    state.  dlog_g of token r is 0 and nothing reaches the initial state from
    after r."""
    rng = np.random.default_rng(31)
    T, r, dk, dv = 9, 4, 3, 3
    x, d_out, d_final = problem(rng, 1, T, 1, dk, dv)
    x["log_g"][0, r] = -np.inf
    g = bwd(x, d_out, d_final, scale=0.6)
    pre = {n: (a[:, :r] if n != "init_state" else a) for n, a in x.items()}
    suf = {n: (a[:, r:] if n != "init_state" else np.zeros_like(a)) for n, a in x.items()}
    gp = bwd(pre, d_out[:, :r], None, scale=0.6)
    gs = bwd(suf, d_out[:, r:], d_final, scale=0.6)
    for key in ("dq", "dk", "dv", "dlog_g", "dbeta"):
        np.testing.assert_allclose(g[key][:, :r], gp[key], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g[key][:, r:], gs[key], rtol=1e-13, atol=1e-13)
    assert np.all(g["dlog_g"][0, r] == 0)
    np.testing.assert_allclose(g["d_init_state"], gp["d_init_state"], rtol=1e-13, atol=1e-13)


def test_B4_packed_equals_separate_documents():
    rng = np.random.default_rng(41)
    lens = [5, 0, 12, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, dk, dv = 2, 5, 4
    x, d_out, d_final = problem(rng, 1, sum(lens), H, dk, dv, N=len(lens))
    g = bwd(x, d_out, d_final, cu_seqlens=cu, scale=0.5)
    for n, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        xn = {m: (t[:, a:e] if m != "init_state" else t[n:n + 1]) for m, t in x.items()}
        gn = bwd(xn, d_out[:, a:e], d_final[n:n + 1], scale=0.5)
        for key in ("dq", "dk", "dv", "dlog_g", "dbeta"):
            np.testing.assert_array_equal(g[key][:, a:e], gn[key])
        np.testing.assert_array_equal(g["d_init_state"][n], gn["d_init_state"][0])


def test_B4_dense_equals_packed():
    rng = np.random.default_rng(42)
    B, T, H, dk, dv = 3, 8, 2, 3, 4
    x, d_out, d_final = problem(rng, B, T, H, dk, dv)
    g = bwd(x, d_out, d_final, scale=1.0)
    flat = {m: (t.reshape((1, B * T) + t.shape[2:]) if m != "init_state" else t) for m, t in x.items()}
    gp = bwd(flat, d_out.reshape(1, B * T, H, dv), d_final, cu_seqlens=np.arange(B + 1) * T, scale=1.0)
    for key in g:
        np.testing.assert_array_equal(g[key].reshape(gp[key].shape), gp[key])


def test_B5_linear_in_the_upstream_gradients():
    rng = np.random.default_rng(51)
    x, do1, df1 = problem(rng, 2, 10, 2, 4, 3)
    _, do2, df2 = problem(rng, 2, 10, 2, 4, 3)
    a, c = 0.75, -1.5
    g1, g2 = bwd(x, do1, df1), bwd(x, do2, df2)
    g = bwd(x, a * do1 + c * do2, a * df1 + c * df2)
    for key in g:
        np.testing.assert_allclose(g[key], a * g1[key] + c * g2[key], rtol=1e-11, atol=1e-11)
    z = bwd(x, None, None)
    assert all(np.all(z[key] == 0) for key in z)


def test_B5_threads_do_not_change_results():
    rng = np.random.default_rng(52)
    x, d_out, d_final = problem(rng, 3, 20, 3, 6, 5)
    a = bwd(x, d_out, d_final, n_threads=1)
    b = bwd(x, d_out, d_final, n_threads=4)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


# --------------------------------------------------------------------------- chunk algebra of the backward
@pytest.mark.parametrize("C", [1, 5, 16, 64])
@pytest.mark.parametrize("dk,dv,T,gate", [(8, 6, 37, 0.1), (16, 16, 130, 0.5), (12, 20, 90, 2.0)])
def test_B6_chunked_backward_equals_token_loop(C, dk, dv, T, gate):
    """The chunk-form reverse mode (the algebra the GPU backward evaluates)
    equals the oracle's token-by-token reverse mode."""
    from chunk_ref import chunk_backward
    rng = np.random.default_rng(C * 13 + dk)
    x, d_out, d_final = problem(rng, 1, T, 1, dk, dv, gate=gate)
    x["beta"] = rng.uniform(0, 1, x["beta"].shape)
    g = bwd(x, d_out, d_final, scale=dk ** -0.5)
    one = lambda a: a[0, :, 0]
    got = chunk_backward(one(x["q"]), one(x["k"]), one(x["v"]), one(x["log_g"]), one(x["beta"]),
                         x["init_state"][0, 0], dk ** -0.5, C, one(d_out), d_final[0, 0])
    for name, a in zip(("dq", "dk", "dv", "dlog_g", "dbeta"), got[:5]):
        ref = one(g[name])
        assert np.abs(a - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max()), name
    ref = g["d_init_state"][0, 0]
    assert np.abs(got[5] - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())
