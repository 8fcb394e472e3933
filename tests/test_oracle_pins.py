"""Pins of the fp64 oracle against what the definition fixes (CPU only).

The oracle is the token loop of the gated delta rule (GLM-5.3-Flash model
notes, Glm5NextTextLinearAttention snippet), with the output read from the
updated state and packed documents reset at their boundaries (NeMo
glm5_next.layers, ``_torch_recurrent_kda``).  None of these checks re-types the
oracle's loop: they use hand-worked examples, closed forms, an exact rational
product-form brute force, a chunked (WY) evaluation and structural invariants.

``KDA_ORACLE_LIB`` may name another compiled oracle library; the mutation test
uses it to show that planted mistakes fail these pins.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bruteforce import run as brute_run
from chunk_ref import chunk_forward

_LIB = oracle.load(os.environ["KDA_ORACLE_LIB"]) if os.environ.get("KDA_ORACLE_LIB") else None
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fwd(*a, **kw):
    return oracle.kda_forward(*a, lib=_LIB, **kw)


def rand_inputs(rng, B, T, H, dk, dv, gate=0.1, beta_lo=0.0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.logaddexp(0, rng.standard_normal((B, T, H, dk))) * gate
    b = beta_lo + (1 - beta_lo) / (1 + np.exp(-rng.standard_normal((B, T, H))))
    return q, k, v, g, b


def rel(x, ref):
    return np.abs(x - ref).max() / max(np.sqrt(np.mean(ref ** 2)), 1e-300)


# --------------------------------------------------------------------------- golden
def _parse_golden(path):
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, rhs = (s.strip() for s in line.split("="))
        out = []
        for tok in rhs.split():
            if tok.startswith("ln("):
                out.append(math.log(float(Fraction(tok[3:-1]))))
            else:
                out.append(float(Fraction(tok)))
        vals[key] = out
    return vals


@pytest.mark.parametrize("name", ["hand_dk2_dv1.txt", "hand_dk1_dv2.txt"])
def test_golden_hand_examples(name):
    g = _parse_golden(os.path.join(GOLDEN, name))
    dk, dv = int(g["dk"][0]), int(g["dv"][0])
    T = len([key for key in g if key.startswith("k.")])
    q = np.array([g[f"q.{t}"] for t in range(T)]).reshape(1, T, 1, dk)
    k = np.array([g[f"k.{t}"] for t in range(T)]).reshape(1, T, 1, dk)
    v = np.array([g[f"v.{t}"] for t in range(T)]).reshape(1, T, 1, dv)
    lg = np.array([g[f"log_g.{t}"] for t in range(T)]).reshape(1, T, 1, dk)
    b = np.array([g[f"beta.{t}"][0] for t in range(T)]).reshape(1, T, 1)
    s0 = np.array(g["init_state"]).reshape(1, 1, dk, dv)
    out, fin = fwd(q, k, v, lg, b, init_state=s0, scale=g["scale"][0])
    exp_out = np.array([g[f"out.{t}"] for t in range(T)]).reshape(1, T, 1, dv)
    np.testing.assert_allclose(out, exp_out, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fin.reshape(-1), g["final_state"], rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("dk,dv", [(3, 5), (8, 8), (16, 4)])
def test_I1_identity_tokens(dk, dv):
    """beta = 0 and log_g = 0: the state is untouched, o_t = scale * S0^T q_t."""
    rng = np.random.default_rng(1)
    q, k, v, _, _ = rand_inputs(rng, 2, 9, 3, dk, dv)
    lg = np.zeros_like(q)
    b = np.zeros(q.shape[:3])
    s0 = rng.standard_normal((2, 3, dk, dv))
    out, fin = fwd(q, k, v, lg, b, init_state=s0, scale=0.7)
    assert np.array_equal(fin, s0)
    expect = 0.7 * np.einsum("bhij,bthi->bthj", s0, q)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-13)


@pytest.mark.parametrize("dk,dv,T", [(8, 3, 8), (16, 16, 11), (6, 9, 4)])
def test_I2_orthonormal_keys_recall(dk, dv, T):
    """beta = 1, no decay, orthonormal keys: S_t^T k_s = v_s for s <= t,
    S_T = (I - sum k k^T) S0 + sum k v^T, and q_t = k_t gives o_t = scale v_t."""
    rng = np.random.default_rng(2)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :T].T                                  # T orthonormal rows
    k = keys.reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    s0 = rng.standard_normal((1, 1, dk, dv))
    lg = np.zeros((1, T, 1, dk))
    b = np.ones((1, T, 1))
    out, fin = fwd(k, k, v, lg, b, init_state=s0, scale=0.5)
    np.testing.assert_allclose(out[0, :, 0], 0.5 * v[0, :, 0], atol=1e-12)
    proj = np.eye(dk) - keys.T @ keys
    np.testing.assert_allclose(fin[0, 0], proj @ s0[0, 0] + keys.T @ v[0, :, 0], atol=1e-12)
    # every earlier key is still recalled by the final state
    np.testing.assert_allclose(keys @ fin[0, 0], v[0, :, 0], atol=1e-12)
    # a fresh query outside the key span reads only the untouched part of S0
    if T < dk:
        qn = Qm[:, T]
        q = np.broadcast_to(qn, (1, T, 1, dk)).copy()
        out2, _ = fwd(q, k, v, lg, b, init_state=s0, scale=1.0)
        np.testing.assert_allclose(out2[0, -1, 0], s0[0, 0].T @ qn, atol=1e-12)


@pytest.mark.parametrize("dk,dv", [(4, 7), (16, 16)])
def test_I3_full_decay_resets(dk, dv):
    """log_g = -inf: the state is wiped each token, S_t = beta_t k_t v_t^T and
    o_t = scale beta_t (q_t . k_t) v_t."""
    rng = np.random.default_rng(3)
    q, k, v, _, b = rand_inputs(rng, 1, 6, 2, dk, dv)
    k = rng.standard_normal(k.shape)                     # not normalised on purpose
    lg = np.full_like(q, -np.inf)
    s0 = rng.standard_normal((1, 2, dk, dv))
    out, fin = fwd(q, k, v, lg, b, init_state=s0, scale=0.3)
    qk = np.einsum("bthi,bthi->bth", q, k)
    np.testing.assert_allclose(out, 0.3 * (b * qk)[..., None] * v, rtol=1e-13, atol=1e-13)
    expect = b[0, -1][:, None, None] * k[0, -1][:, :, None] * v[0, -1][:, None, :]
    np.testing.assert_allclose(fin[0], expect, rtol=1e-13, atol=1e-13)


def test_scalar_closed_form():
    """dk = dv = 1: s_t = a s' + beta k (v - a s' k)... written as
    s_t = a_t s_{t-1} (1 - beta_t k_t^2) + beta_t k_t v_t, o_t = scale q_t s_t."""
    rng = np.random.default_rng(4)
    T = 12
    q, k, v = (rng.standard_normal((1, T, 1, 1)) for _ in range(3))
    lg = -rng.uniform(0, 2, (1, T, 1, 1))
    b = rng.uniform(0, 1, (1, T, 1))
    out, fin = fwd(q, k, v, lg, b, init_state=np.array([[[[0.25]]]]), scale=1.5)
    s = 0.25
    for t in range(T):
        a, kk, vv, bb = math.exp(lg[0, t, 0, 0]), k[0, t, 0, 0], v[0, t, 0, 0], b[0, t, 0]
        s = a * s * (1 - bb * kk * kk) + bb * kk * vv
        assert abs(out[0, t, 0, 0] - 1.5 * q[0, t, 0, 0] * s) < 1e-13
    assert abs(fin[0, 0, 0, 0] - s) < 1e-13


# --------------------------------------------------------------------------- brute force
def _dyadic(rng, shape, choices):
    return np.array([Fraction(choices[i]) for i in rng.integers(0, len(choices), size=int(np.prod(shape)))],
                    dtype=object).reshape(shape)


@pytest.mark.parametrize("dk,dv,T,seed", [(3, 4, 8, 0), (4, 4, 7, 1), (4, 3, 5, 2), (2, 4, 8, 3)])
def test_I4_bruteforce_exact(dk, dv, T, seed):
    """Exact rational product form (transition matrices) vs the fp64 token loop."""
    rng = np.random.default_rng(seed)
    alphas = ["1", "1/2", "3/4", "1/8", "7/8"]
    vals = ["-1", "-1/2", "-1/4", "0", "1/4", "1/2", "3/4", "1", "3/2"]
    alpha = _dyadic(rng, (T, dk), alphas)
    k = _dyadic(rng, (T, dk), vals)
    q = _dyadic(rng, (T, dk), vals)
    v = _dyadic(rng, (T, dv), vals)
    beta = _dyadic(rng, (T,), ["0", "1/4", "1/2", "3/4", "1"])
    S0 = _dyadic(rng, (dk, dv), vals)
    scale = Fraction(1, 2)
    ex_out, ex_S = brute_run(alpha.tolist(), list(beta), k.tolist(), v.tolist(), q.tolist(),
                             S0.tolist(), scale)
    f = np.vectorize(float)
    out, fin = fwd(f(q).reshape(1, T, 1, dk), f(k).reshape(1, T, 1, dk), f(v).reshape(1, T, 1, dv),
                   np.log(f(alpha)).reshape(1, T, 1, dk), f(beta).reshape(1, T, 1),
                   init_state=f(S0).reshape(1, 1, dk, dv), scale=0.5)
    ex_out = f(np.array(ex_out, dtype=object))
    ex_S = f(np.array(ex_S, dtype=object))
    tol = 1e-13 * max(1.0, np.abs(ex_out).max(), np.abs(ex_S).max())
    np.testing.assert_allclose(out[0, :, 0], ex_out, rtol=0, atol=tol)
    np.testing.assert_allclose(fin[0, 0], ex_S, rtol=0, atol=tol)


# --------------------------------------------------------------------------- chunk algebra
@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("dk,dv,T,gate", [(8, 6, 37, 0.1), (16, 16, 130, 0.5), (32, 24, 200, 2.0)])
def test_I5_chunked_equals_token_loop(C, dk, dv, T, gate):
    rng = np.random.default_rng(C * 7 + dk)
    q, k, v, g, b = rand_inputs(rng, 1, T, 1, dk, dv, gate=gate)
    s0 = rng.standard_normal((1, 1, dk, dv)) * 0.1
    out, fin = fwd(q, k, v, g, b, init_state=s0, scale=dk ** -0.5)
    co, cs = chunk_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], b[0, :, 0], s0[0, 0],
                           dk ** -0.5, C)
    assert rel(co, out[0, :, 0]) < 1e-10
    assert rel(cs, fin[0, 0]) < 1e-10


# --------------------------------------------------------------------------- invariants
def test_I6_packed_equals_separate_documents():
    rng = np.random.default_rng(6)
    lens = [5, 0, 17, 1, 64, 30]
    T, H, dk, dv = sum(lens), 3, 8, 5
    q, k, v, g, b = rand_inputs(rng, 1, T, H, dk, dv, gate=0.3)
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, fin = fwd(q, k, v, g, b, init_state=s0, cu_seqlens=cu, scale=0.4)
    for n, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        sl = slice(a, e)
        o1, f1 = fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], b[:, sl], init_state=s0[n:n + 1], scale=0.4)
        np.testing.assert_array_equal(out[:, sl], o1)
        np.testing.assert_array_equal(fin[n], f1[0])
    # zero initial states when none is given
    out0, fin0 = fwd(q, k, v, g, b, cu_seqlens=cu, scale=0.4)
    o2, f2 = fwd(q[:, :5], k[:, :5], v[:, :5], g[:, :5], b[:, :5], init_state=np.zeros((1, H, dk, dv)),
                 scale=0.4)
    np.testing.assert_array_equal(out0[:, :5], o2)
    assert np.all(fin0[1] == 0)                          # empty document keeps its zero state


def test_I6_dense_batch_equals_packed():
    rng = np.random.default_rng(61)
    B, T, H, dk, dv = 3, 20, 2, 4, 6
    q, k, v, g, b = rand_inputs(rng, B, T, H, dk, dv)
    s0 = rng.standard_normal((B, H, dk, dv))
    out, fin = fwd(q, k, v, g, b, init_state=s0, scale=1.0)
    flat = [x.reshape((1, B * T) + x.shape[2:]) for x in (q, k, v, g, b)]
    cu = np.arange(B + 1) * T
    out2, fin2 = fwd(*flat, init_state=s0, cu_seqlens=cu, scale=1.0)
    np.testing.assert_array_equal(out.reshape(out2.shape), out2)
    np.testing.assert_array_equal(fin, fin2)


@pytest.mark.parametrize("split", [1, 13, 64, 99])
def test_I7_resume_from_final_state(split):
    rng = np.random.default_rng(7)
    T, H, dk, dv = 100, 2, 8, 8
    q, k, v, g, b = rand_inputs(rng, 2, T, H, dk, dv)
    s0 = rng.standard_normal((2, H, dk, dv))
    out, fin = fwd(q, k, v, g, b, init_state=s0)
    a = slice(0, split)
    c = slice(split, T)
    o1, f1 = fwd(q[:, a], k[:, a], v[:, a], g[:, a], b[:, a], init_state=s0)
    o2, f2 = fwd(q[:, c], k[:, c], v[:, c], g[:, c], b[:, c], init_state=f1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(f2, fin, rtol=0, atol=1e-13)


def test_I8_linear_in_v_and_state():
    rng = np.random.default_rng(8)
    T, H, dk, dv = 40, 2, 6, 5
    q, k, v1, g, b = rand_inputs(rng, 1, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, dk, dv))
    s2 = rng.standard_normal((1, H, dk, dv))
    a, c = 0.75, -1.25
    o1, f1 = fwd(q, k, v1, g, b, init_state=s1)
    o2, f2 = fwd(q, k, v2, g, b, init_state=s2)
    o3, f3 = fwd(q, k, a * v1 + c * v2, g, b, init_state=a * s1 + c * s2)
    np.testing.assert_allclose(o3, a * o1 + c * o2, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + c * f2, atol=1e-12)
    # permuting the value columns of v and S0 permutes o and S
    perm = rng.permutation(dv)
    o4, f4 = fwd(q, k, v1[..., perm], g, b, init_state=s1[..., perm])
    np.testing.assert_array_equal(o4, o1[..., perm])
    np.testing.assert_array_equal(f4, f1[..., perm])


def test_decode_rows_in_order():
    """Verify: n_tok rows applied in order equal single-row calls chained
    (metrale glm5next_layer: verify row t uses slot t)."""
    rng = np.random.default_rng(9)
    N, n_tok, H, dk, dv = 3, 4, 2, 8, 8
    q, k, v, g, b = rand_inputs(rng, N, n_tok, H, dk, dv)
    s = rng.standard_normal((N, H, dk, dv))
    out, fin = oracle.kda_step(q, k, v, g, b, s) if _LIB is None else fwd(q, k, v, g, b, init_state=s)
    st = s
    for t in range(n_tok):
        sl = slice(t, t + 1)
        o1, st = fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], b[:, sl], init_state=st)
        np.testing.assert_allclose(o1, out[:, sl], rtol=0, atol=1e-13)
    np.testing.assert_allclose(st, fin, rtol=0, atol=1e-13)
    # swapping two rows changes the result (the order matters)
    qs, ks, vs, gs, bs = (np.concatenate([x[:, 1:2], x[:, 0:1], x[:, 2:]], axis=1) for x in (q, k, v, g, b))
    _, fin_sw = fwd(qs, ks, vs, gs, bs, init_state=s)
    assert np.abs(fin_sw - fin).max() > 1e-6


def test_threads_do_not_change_results():
    rng = np.random.default_rng(10)
    q, k, v, g, b = rand_inputs(rng, 4, 33, 5, 8, 8)
    o1, f1 = fwd(q, k, v, g, b, n_threads=1)
    o2, f2 = fwd(q, k, v, g, b, n_threads=4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_rejects_bad_cu_seqlens():
    rng = np.random.default_rng(11)
    q, k, v, g, b = rand_inputs(rng, 1, 10, 1, 4, 4)
    with pytest.raises(ValueError):
        fwd(q, k, v, g, b, cu_seqlens=np.array([0, 6, 4, 10]))
    with pytest.raises(ValueError):
        fwd(q, k, v, g, b, cu_seqlens=np.array([0, 4, 9]))
