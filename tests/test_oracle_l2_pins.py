"""Pins of the oracle's optional L2 normalisation of q and k (CPU only).

The pages print no normalisation step; the reading taken is the plain one:
each (token, head) row of q and of k divided by sqrt(sum of squares + eps),
before the recurrence.  The pins are closed forms and invariances, not the
formula retyped: the squared norm of a normalised row, ratios and signs kept,
a one-hot row with eps, the zero row, per-row independence, and the
recurrence's invariance to per-row positive rescaling of q and k once they are
normalised.

``KDA_ORACLE_LIB`` may name another compiled oracle library; the mutation test
uses it to show that planted mistakes fail these pins.
"""
import os

import numpy as np

import oracle

_LIB = oracle.load(os.environ["KDA_ORACLE_LIB"]) if os.environ.get("KDA_ORACLE_LIB") else None


def l2(q, k, eps):
    return oracle.qk_l2norm(q, k, eps, lib=_LIB)


def test_L1_squared_norm_of_a_normalised_row():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 3, 16)) * 4.0
    k = rng.standard_normal((5, 3, 16)) * 0.1
    for eps in (0.0, 1e-3):
        qn, kn = l2(q, k, eps)
        for x, xn in ((q, qn), (k, kn)):
            ss = np.sum(x ** 2, axis=-1)
            np.testing.assert_allclose(np.sum(xn ** 2, axis=-1), ss / (ss + eps), rtol=1e-13)


def test_L2_ratios_and_signs_kept():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((7, 8)) + 0.5
    k = rng.standard_normal((7, 8)) - 0.5
    qn, kn = l2(q, k, 1e-6)
    for x, xn in ((q, qn), (k, kn)):
        np.testing.assert_allclose(xn / xn[:, :1], x / x[:, :1], rtol=1e-12)
        assert np.all(np.sign(xn) == np.sign(x))


def test_L3_one_hot_row_with_eps_and_zero_row():
    D, c, eps = 16, 0.05, 1e-3
    x = np.zeros((2, D))
    x[0, 3] = c
    x[1, 11] = -2.0 * c
    qn, kn = l2(x, x[::-1].copy(), eps)
    np.testing.assert_allclose(qn[0, 3], c / np.sqrt(c * c + eps), rtol=1e-14)
    np.testing.assert_allclose(qn[1, 11], -2 * c / np.sqrt(4 * c * c + eps), rtol=1e-14)
    np.testing.assert_allclose(kn[1, 3], c / np.sqrt(c * c + eps), rtol=1e-14)
    assert np.count_nonzero(qn) == 2 and np.count_nonzero(kn) == 2
    zq, zk = l2(np.zeros((3, D)), np.zeros((3, D)), 1e-6)
    assert np.all(zq == 0.0) and np.all(zk == 0.0)


def test_L4_rows_are_independent_and_the_axis_is_head_dim():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 5, 3, 8))
    k = rng.standard_normal((2, 5, 3, 8))
    qn, kn = l2(q, k, 1e-6)
    for b in range(2):
        for t in range(5):
            for h in range(3):
                a, c = l2(q[b, t, h][None], k[b, t, h][None], 1e-6)
                np.testing.assert_array_equal(a[0], qn[b, t, h])
                np.testing.assert_array_equal(c[0], kn[b, t, h])
    # rescaling one row leaves every row unchanged at eps = 0
    q2 = q.copy()
    q2[1, 2, 0] *= 7.0
    np.testing.assert_allclose(l2(q2, k, 0.0)[0], l2(q, k, 0.0)[0], rtol=1e-14)


def test_L5_recurrence_invariant_to_row_rescaling_of_q_and_k():
    """With normalisation (eps = 0) the recurrence sees only the directions of
    the q and k rows: positive per-row factors on q and on k, drawn
    independently, change nothing; on rows that are already unit vectors the
    normalised run equals the plain run."""
    from kda_inputs import make_inputs, to_f64
    inp = make_inputs(B=1, T=40, H=2, dk=5, dv=3, dtype="f32", seed=7, lengths=[17, 0, 23],
                      init="normal", init_std=0.3)
    q, k, v, g, b = (to_f64(inp[n]) for n in ("q", "k", "v", "log_g", "beta"))
    s0, cu = to_f64(inp["init_state"]), inp["cu_seqlens"].numpy()
    rng = np.random.default_rng(8)
    cq = rng.uniform(0.1, 10.0, q.shape[:-1] + (1,))
    ck = rng.uniform(0.1, 10.0, k.shape[:-1] + (1,))
    run = lambda qq, kk, eps: oracle.kda_forward(qq, kk, v, g, b, init_state=s0, cu_seqlens=cu,
                                                 qk_l2norm_eps=eps, lib=_LIB)
    o1, f1 = run(q, k, 0.0)
    o2, f2 = run(q * cq, k * ck, 0.0)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(f2, f1, rtol=1e-11, atol=1e-13)
    qu = q / np.linalg.norm(q, axis=-1, keepdims=True)
    ku = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o3, f3 = oracle.kda_forward(qu, ku, v, g, b, init_state=s0, cu_seqlens=cu, lib=_LIB)
    np.testing.assert_allclose(o1, o3, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(f1, f3, rtol=1e-11, atol=1e-13)
    # and it is not the identity on rows that are not unit vectors
    o4, _ = oracle.kda_forward(q * cq, k * ck, v, g, b, init_state=s0, cu_seqlens=cu, lib=_LIB)
    assert np.abs(o4 - o1).max() > 1e-3
