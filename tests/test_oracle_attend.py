"""Pins of the oracle's decode-step attention (gist.science/nl "Technische
Samenvatting", "Memory en Latentie": attention read over the decoded cache).

The oracle is the plain definition softmax(scale q k^T) v in fp64; it is
checked against scipy's softmax with a numpy weighted sum, closed forms
(uniform scores give the mean of v, one token gives that token, a dominant key
gives its value), token-permutation invariance and the empty case.  CPU only.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as O


@pytest.mark.parametrize("T,D,G,scale", [(1, 16, 1, 0.5), (7, 64, 4, 0.125), (300, 128, 4, 0.088),
                                         (33, 256, 16, 1.0)])
def test_attend_matches_scipy_softmax(T, D, G, scale):
    rng = np.random.default_rng(T * 131 + D)
    k = rng.normal(size=(T, D)) * rng.lognormal(0.0, 0.5, size=D)
    v = rng.normal(size=(T, D))
    q = rng.normal(size=(G, D))
    ref = np.stack([softmax(scale * (k @ q[g])) @ v for g in range(G)])
    np.testing.assert_allclose(O.attend(k, v, q, scale), ref, rtol=1e-12, atol=1e-12)


def test_uniform_scores_give_the_mean_of_v():
    rng = np.random.default_rng(1)
    k = rng.normal(size=(40, 32))
    v = rng.normal(size=(40, 32))
    out = O.attend(k, v, np.zeros((2, 32)), 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), (2, 32)), rtol=0, atol=1e-14)


def test_one_token_gives_its_value():
    rng = np.random.default_rng(2)
    k, v, q = rng.normal(size=(1, 64)), rng.normal(size=(1, 64)), rng.normal(size=(3, 64))
    np.testing.assert_allclose(O.attend(k, v, q, 3.0), np.repeat(v, 3, axis=0), rtol=0, atol=1e-15)


def test_dominant_key_gives_its_value():
    rng = np.random.default_rng(3)
    T, D = 50, 64
    k = rng.normal(size=(T, D)) * 0.01
    v = rng.normal(size=(T, D))
    j = 17
    k[j] = 1.0
    q = np.ones((1, D))
    # score gap >= 64 * (1 - 0.05) * scale: weights of the others below e^-60
    out = O.attend(k, v, q, 1.0)
    np.testing.assert_allclose(out[0], v[j], rtol=0, atol=1e-20 + 1e-12)


def test_token_order_does_not_matter():
    rng = np.random.default_rng(4)
    k, v, q = rng.normal(size=(60, 32)), rng.normal(size=(60, 32)), rng.normal(size=(4, 32))
    perm = rng.permutation(60)
    np.testing.assert_allclose(O.attend(k, v, q, 0.4), O.attend(k[perm], v[perm], q, 0.4),
                               rtol=1e-13, atol=1e-14)


def test_query_rows_are_independent():
    rng = np.random.default_rng(5)
    k, v, q = rng.normal(size=(20, 16)), rng.normal(size=(20, 16)), rng.normal(size=(3, 16))
    full = O.attend(k, v, q, 0.9)
    for g in range(3):
        np.testing.assert_array_equal(full[g], O.attend(k, v, q[g:g + 1], 0.9)[0])


def test_empty_sequence_gives_zeros():
    out = O.attend(np.zeros((0, 32)), np.zeros((0, 32)), np.ones((2, 32)), 1.0)
    assert out.shape == (2, 32) and not out.any()
