"""Pins of the oracle's short causal depthwise convolution (CPU only).

The convolution that feeds q, k and v (NeMo glm5_next.layers,
``_TorchShortConvolution``: depthwise causal Conv1d over [batch, sequence,
channels], reset at packed boundaries).  None of these re-types the oracle's
loop: numpy's own convolution, impulse responses, packed versus separate
documents, resume from the cache at any split, and closed forms for K = 1 and
the SiLU option.

``KDA_ORACLE_LIB`` may name another compiled oracle library; the mutation test
uses it to show that planted mistakes fail these pins.
"""
import os

import numpy as np
import pytest

import oracle

_LIB = oracle.load(os.environ["KDA_ORACLE_LIB"]) if os.environ.get("KDA_ORACLE_LIB") else None


def conv(x, w, **kw):
    return oracle.short_conv(x, w, lib=_LIB, **kw)


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7])
def test_C1_equals_numpy_convolution(K):
    rng = np.random.default_rng(K)
    x = rng.standard_normal((2, 37, 5))
    w = rng.standard_normal((5, K))
    y, fin = conv(x, w)
    for b in range(2):
        for c in range(5):
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:37]     # causal, zeros before the start
            np.testing.assert_allclose(y[b, :, c], ref, rtol=1e-13, atol=1e-13)
            np.testing.assert_array_equal(fin[b, c], x[b, 37 - (K - 1):, c] if K > 1 else np.zeros(0))


def test_C2_impulse_responses_stop_at_the_document_end():
    K, Cn = 4, 3
    w = np.arange(1, 1 + Cn * K, dtype=np.float64).reshape(Cn, K)
    lens = [6, 5]
    cu = np.array([0, 6, 11])
    x = np.zeros((1, 11, Cn))
    x[0, 4, :] = 1.0                      # two tokens before the end of document 0
    y, _ = conv(x, w, cu_seqlens=cu)
    for c in range(Cn):
        # y[4 + m] = w[c, K-1-m] while inside document 0; nothing in document 1
        np.testing.assert_array_equal(y[0, :4, c], 0.0)
        np.testing.assert_array_equal(y[0, 4:6, c], [w[c, 3], w[c, 2]])
        np.testing.assert_array_equal(y[0, 6:, c], 0.0)


def test_C3_packed_equals_separate_documents():
    rng = np.random.default_rng(3)
    K, Cn = 4, 6
    lens = [5, 0, 2, 17, 1, 0, 9]          # empty documents and ones shorter than K - 1
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((1, sum(lens), Cn))
    w = rng.standard_normal((Cn, K))
    c0 = rng.standard_normal((len(lens), Cn, K - 1))
    y, fin = conv(x, w, cu_seqlens=cu, init_cache=c0)
    for n, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        yn, fn = conv(x[:, a:e], w, init_cache=c0[n:n + 1])
        np.testing.assert_array_equal(y[:, a:e], yn)
        np.testing.assert_array_equal(fin[n], fn[0])
    np.testing.assert_array_equal(fin[1], c0[1])                           # empty: cache unchanged
    np.testing.assert_array_equal(fin[2], np.concatenate([c0[2][:, 2:], x[0, 5:7].T], axis=1))  # 2 < K - 1


@pytest.mark.parametrize("split", [1, 2, 3, 10, 29])
def test_C4_resume_from_the_cache(split):
    rng = np.random.default_rng(4)
    K, Cn, T = 4, 5, 30
    x = rng.standard_normal((3, T, Cn))
    w = rng.standard_normal((Cn, K))
    c0 = rng.standard_normal((3, Cn, K - 1))
    y, fin = conv(x, w, init_cache=c0)
    y1, f1 = conv(x[:, :split], w, init_cache=c0)
    y2, f2 = conv(x[:, split:], w, init_cache=f1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(f2, fin)


def test_C5_single_tap_and_silu():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 9, 4))
    w1 = rng.standard_normal((4, 1))
    y, fin = conv(x, w1)
    np.testing.assert_allclose(y, x * w1[:, 0], rtol=1e-15, atol=0)
    assert fin.shape == (2, 4, 0)
    w = rng.standard_normal((4, 3))
    z, _ = conv(x, w)
    s, _ = conv(x, w, act=1)
    np.testing.assert_allclose(s, z / (1.0 + np.exp(-z)), rtol=1e-14, atol=1e-14)   # SiLU after the sum


def test_C6_rejects_bad_arguments():
    x = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        conv(x, np.zeros((2, 2)), act=2)
    with pytest.raises(ValueError):
        conv(x, np.zeros((2, 2)), cu_seqlens=np.array([0, 3]))
