"""Pins of the decode-attention oracle (CPU only).

Each pin is fixed by something other than the oracle's own formula: a library
routine (scipy's softmax), a closed form worked by hand, or an invariance of
the attention output.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import attention, qjl


def _random_case(rng, G=2, n_q=3, n_k=37, m=64, d_v=8):
    bits = rng.integers(0, 2**32, size=(G * n_k, m // 32), dtype=np.uint64).astype(np.uint32)
    norms = rng.uniform(0.5, 3.0, size=G * n_k)
    Sq = rng.standard_normal((G * n_q, m))
    V = rng.standard_normal((G * n_k, d_v))
    return Sq, bits, norms, V


def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7, 33)) * 30
    np.testing.assert_allclose(attention.softmax_rows(x), scipy.special.softmax(x, axis=-1),
                               rtol=1e-12, atol=1e-300)


def test_softmax_shift_invariant_and_safe():
    x = np.array([[1000.0, 999.0, -5.0]])
    a = attention.softmax_rows(x)
    assert np.all(np.isfinite(a))
    np.testing.assert_allclose(a, attention.softmax_rows(x - 1000.0), rtol=1e-13)


def test_matches_scipy_pipeline():
    """Scores from the estimator, weights from scipy, output by matrix product."""
    rng = np.random.default_rng(1)
    G, n_q, n_k, m, d_v = 2, 3, 37, 64, 8
    Sq, bits, norms, V = _random_case(rng, G, n_q, n_k, m, d_v)
    out = attention.decode_attention(Sq, bits, norms, V, m, 0.0, 0.3, G, n_q, n_k)
    s = qjl.score(Sq, bits, norms, m, 0.0, G, n_q, n_k)
    for g in range(G):
        a = scipy.special.softmax(0.3 * s[g], axis=-1)
        np.testing.assert_allclose(out[g], a @ V[g * n_k:(g + 1) * n_k], rtol=1e-12, atol=1e-12)


def test_two_keys_closed_form():
    """Two keys, scores worked out by hand: weight of key 0 is 1/(1+e^(tau(s1-s0)))."""
    m, d_v, tau = 32, 3, 0.25
    # key 0: all bits 1 (every sign +), key 1: all bits 0 (every sign -)
    bits = np.array([[0xFFFFFFFF], [0x00000000]], dtype=np.uint32)
    norms = np.array([2.0, 1.0])
    Sq = np.full((1, m), 0.5)              # sum_j Sq_j = 16
    c = math.sqrt(math.pi / 2) / m
    s0, s1 = c * 2.0 * 16.0, -c * 1.0 * 16.0
    w0 = 1.0 / (1.0 + math.exp(tau * (s1 - s0)))
    V = np.array([[1.0, -2.0, 0.5], [4.0, 3.0, -1.0]])
    out = attention.decode_attention(Sq, bits, norms, V, m, 0.0, tau, 1, 1, 2)
    np.testing.assert_allclose(out[0, 0], w0 * V[0] + (1 - w0) * V[1], rtol=1e-14)


@pytest.mark.parametrize("how", ["zero_norms", "zero_scale"])
def test_uniform_weights_give_mean(how):
    rng = np.random.default_rng(2)
    G, n_q, n_k, m, d_v = 2, 2, 29, 64, 5
    Sq, bits, norms, V = _random_case(rng, G, n_q, n_k, m, d_v)
    scale = 0.7
    if how == "zero_norms":
        norms = np.zeros_like(norms)
    else:
        scale = 0.0
    out = attention.decode_attention(Sq, bits, norms, V, m, 0.0, scale, G, n_q, n_k)
    for g in range(G):
        mean = V[g * n_k:(g + 1) * n_k].mean(axis=0)
        for i in range(n_q):
            np.testing.assert_allclose(out[g, i], mean, rtol=1e-13, atol=1e-14)


def test_key_permutation_invariance():
    rng = np.random.default_rng(3)
    G, n_q, n_k, m, d_v = 1, 2, 41, 64, 6
    Sq, bits, norms, V = _random_case(rng, G, n_q, n_k, m, d_v)
    perm = rng.permutation(n_k)
    a = attention.decode_attention(Sq, bits, norms, V, m, 0.0, 0.2, G, n_q, n_k)
    b = attention.decode_attention(Sq, bits[perm], norms[perm], V[perm], m, 0.0, 0.2, G, n_q, n_k)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_dominant_key_returns_its_value():
    """One key whose score exceeds every other by a wide margin takes all the weight."""
    rng = np.random.default_rng(4)
    n_k, m, d_v = 16, 64, 4
    Sq = np.abs(rng.standard_normal((1, m)))  # all positive
    bits = np.zeros((n_k, m // 32), dtype=np.uint32)
    bits[5] = 0xFFFFFFFF                       # key 5: every sign +, so its score is the largest
    norms = np.ones(n_k)
    norms[5] = 50.0
    V = rng.standard_normal((n_k, d_v))
    out = attention.decode_attention(Sq, bits, norms, V, m, 0.0, 1.0, 1, 1, n_k)
    np.testing.assert_allclose(out[0, 0], V[5], rtol=0, atol=1e-12)
