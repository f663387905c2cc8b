"""Pins of the oracle's quaternion algebra and of the 2T table.

The Hamilton product is checked against the 2x2 complex-matrix
representation; 2T against the definition of the unit Hurwitz quaternions and
the facts the pages print (24 elements, closed group, pairwise angle at
least 60 degrees: the abstract; gist.science/nl technical summary,
Methodologie 1).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
from tests import refmath as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
E = np.eye(4)


def test_qmul_matches_matrix_representation():
    rng = np.random.default_rng(1)
    for _ in range(500):
        a, b = rng.normal(size=4), rng.normal(size=4)
        np.testing.assert_allclose(O.qmul(a, b), R.qprod(a, b), rtol=0, atol=1e-13)


def test_basis_relations():
    one, i, j, k = E
    for u in (i, j, k):
        np.testing.assert_array_equal(O.qmul(u, u), -one)
    np.testing.assert_array_equal(O.qmul(O.qmul(i, j), k), -one)
    np.testing.assert_array_equal(O.qmul(i, j), k)
    np.testing.assert_array_equal(O.qmul(j, i), -k)
    np.testing.assert_array_equal(O.qmul(j, k), i)
    np.testing.assert_array_equal(O.qmul(k, i), j)


def test_norm_multiplicative_and_left_isometry():
    """|a b| = |a| |b|; left multiplication by a unit quaternion preserves
    inner products (the isometry of S^3 the abstract invokes)."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        a, b, c = rng.normal(size=(3, 4))
        assert abs(np.linalg.norm(O.qmul(a, b)) - np.linalg.norm(a) * np.linalg.norm(b)) < 1e-13 * (
            1 + np.linalg.norm(a) * np.linalg.norm(b))
        u = a / np.linalg.norm(a)
        assert abs(O.qmul(u, b) @ O.qmul(u, c) - b @ c) < 1e-12 * (1 + abs(b @ c))


def test_conjugate_identity():
    """<x, a b> = <conj(a) x, b> for unit a: the identity the encode search
    uses to score all 24 left-products through one transform."""
    rng = np.random.default_rng(3)
    for _ in range(300):
        x, a, b = rng.normal(size=(3, 4))
        a /= np.linalg.norm(a)
        assert abs(x @ O.qmul(a, b) - O.qmul(R.conj(a), x) @ b) < 1e-12


def test_t2_is_the_set_of_hurwitz_units():
    t2 = O.t2_elements()
    assert t2.shape == (24, 4)
    assert len({tuple(r) for r in t2}) == GOLD["primary_group_order"]["value"]
    assert {tuple(r) for r in t2} == set(R.hurwitz_units())


def test_t2_closed_under_product_and_inverse():
    t2 = O.t2_elements()
    S = {tuple(r) for r in t2}
    assert GOLD["primary_is_closed_group"]["value"]
    for a, b in itertools.product(t2, t2):
        assert tuple(O.qmul(a, b)) in S
    for a in t2:
        # the inverse of a unit quaternion is its conjugate, and it is in 2T
        assert tuple(R.conj(a)) in S
        np.testing.assert_array_equal(O.qmul(a, R.conj(a)), E[0])
    assert tuple(-E[0]) in S


def test_t2_gram_values_and_60_degree_neighbours():
    t2 = O.t2_elements()
    G = t2 @ t2.T
    assert set(np.round(G.ravel(), 12)) == {1.0, 0.5, 0.0, -0.5, -1.0}
    off = G[~np.eye(24, dtype=bool)]
    min_angle = np.degrees(np.arccos(off.max()))
    assert abs(min_angle - GOLD["primary_min_pairwise_angle_deg"]["value"]) < 1e-9
    # every vertex of the 24-cell has 8 nearest neighbours
    assert all(int((np.abs(G[p] - 0.5) < 1e-12).sum()) == 8 for p in range(24))


def test_t2_element_order_census():
    """SL(2,3) has 1 element of order 1, 1 of order 2, 8 of order 3, 6 of
    order 4 and 8 of order 6."""
    census = {}
    for a in O.t2_elements():
        p, n = a.copy(), 1
        while not np.array_equal(p, E[0]):
            p, n = O.qmul(p, a), n + 1
            assert n <= 24
        census[n] = census.get(n, 0) + 1
    assert census == {1: 1, 2: 1, 3: 8, 4: 6, 6: 8}


def test_t2_canonical_order():
    """The order of 2T is a reading (the pages give only the set): units
    +1, -1, +i, -i, +j, -j, +k, -k, then (s0, s1, s2, s3)/2 with s_m = -1
    when bit m of p - 8 is set."""
    t2 = O.t2_elements()
    for p in range(8):
        want = np.zeros(4)
        want[p // 2] = 1.0 if p % 2 == 0 else -1.0
        np.testing.assert_array_equal(t2[p], want)
    for p in range(8, 24):
        want = np.array([-0.5 if (p - 8) >> m & 1 else 0.5 for m in range(4)])
        np.testing.assert_array_equal(t2[p], want)


@pytest.mark.parametrize("S", [8, 32])
def test_codeword_count_and_unit_norm(S):
    """24 S effective codewords (192 at S=8, 768 at S=32), all unit."""
    q = O.make_codebook(0, 1, 1, 0, S)[0, 0]
    cw = np.stack([O.codeword(q, k) for k in range(24 * S)])
    assert len(cw) == GOLD["effective_codewords"]["value"][str(S)]
    assert np.abs(np.linalg.norm(cw, axis=1) - 1).max() < 1e-6
    # and they are the products a_p q_s, computed independently
    np.testing.assert_allclose(cw, R.codewords_matrix_rep(q, O.t2_elements()), atol=1e-14)
