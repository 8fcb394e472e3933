"""Pins of the oracle's gated per-head RMSNorm (CPU only).

NeMo glm5_next.layers, ``_TorchRMSNormGated``: normalise [batch, sequence,
heads, head_dim], then gate with a sigmoid; every norm is x * w / rms (metrale
glm5next_layer invariants), never x * (1 + w) / rms.  The pins are closed forms
and invariances, not the formula retyped: unit RMS of the normalised row,
scale invariance, the constant row with eps, the gate's limits and its value
at 0, the per-channel weight, and per-row independence.

``KDA_ORACLE_LIB`` may name another compiled oracle library; the mutation test
uses it to show that planted mistakes fail these pins.
"""
import os

import numpy as np

import oracle

_LIB = oracle.load(os.environ["KDA_ORACLE_LIB"]) if os.environ.get("KDA_ORACLE_LIB") else None
OPEN = 60.0  # sigmoid(60) = 1 to double precision


def norm(o, g, w, eps):
    return oracle.gated_rmsnorm(o, g, w, eps, lib=_LIB)


def test_N1_unit_rms_with_open_gate_and_unit_weight():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((5, 3, 16)) * 7.0
    y = norm(o, np.full(o.shape, OPEN), np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(y ** 2, axis=-1), 1.0, rtol=1e-13)
    # the direction of each row is kept
    np.testing.assert_allclose(y * np.sqrt(np.mean(o ** 2, axis=-1, keepdims=True)), o, rtol=1e-12)


def test_N2_scale_invariant_without_eps():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((4, 32))
    g = rng.standard_normal((4, 32))
    w = rng.standard_normal(32)
    np.testing.assert_allclose(norm(3.5 * o, g, w, 0.0), norm(o, g, w, 0.0), rtol=1e-13, atol=1e-15)


def test_N3_constant_row_and_zero_row_with_eps():
    a, eps, D = 0.3, 0.01, 8
    y = norm(np.full((1, D), a), np.full((1, D), OPEN), np.ones(D), eps)
    np.testing.assert_allclose(y, a / np.sqrt(a * a + eps), rtol=1e-14)
    assert np.all(norm(np.zeros((2, D)), np.zeros((2, D)), np.ones(D), eps) == 0.0)


def test_N4_gate_limits_and_half_at_zero():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((6, 16))
    w = rng.standard_normal(16)
    open_ = norm(o, np.full(o.shape, OPEN), w, 1e-6)
    np.testing.assert_allclose(norm(o, np.zeros(o.shape), w, 1e-6), 0.5 * open_, rtol=1e-14)
    np.testing.assert_allclose(norm(o, np.full(o.shape, -OPEN), w, 1e-6), 0.0, atol=1e-25)
    # the gate acts after the normalisation: a gate that differs across channels leaves the RMS alone
    g = rng.standard_normal(o.shape)
    y = norm(o, g, np.ones(16), 0.0)
    np.testing.assert_allclose(y * (1.0 + np.exp(-g)), norm(o, np.full(o.shape, OPEN), np.ones(16), 0.0),
                               rtol=1e-12)


def test_N5_weight_is_a_plain_per_channel_scale():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 2, 8))
    g = rng.standard_normal(o.shape)
    w = rng.standard_normal(8)
    base = norm(o, g, np.ones(8), 1e-5)
    np.testing.assert_allclose(norm(o, g, w, 1e-5), base * w, rtol=1e-13, atol=1e-16)
    assert np.all(norm(o, g, np.zeros(8), 1e-5) == 0.0)          # w = 0 gives 0, not x (no 1 + w)


def test_N6_rows_are_independent():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((7, 16))
    g = rng.standard_normal((7, 16))
    w = rng.standard_normal(16)
    y = norm(o, g, w, 1e-6)
    for r in range(7):
        np.testing.assert_array_equal(norm(o[r:r + 1], g[r:r + 1], w, 1e-6), y[r:r + 1])
