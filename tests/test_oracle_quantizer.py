"""Pins of the oracle's per-chunk steps: norm, norm code, nearest codeword.

The direction is quantised to the codeword of largest inner product
(gist.science/nl technical summary, Methodologie 1; the abstract).  The pins:
a KD-tree nearest neighbour (scipy) over the codewords built independently,
codeword inputs, the 24-cell's deep hole, and the closed form of the best
2T element.
"""
import numpy as np
import pytest
from scipy.spatial import cKDTree

import oracle as O
from tests import refmath as R


def test_norm2_is_the_declared_fp32_chain():
    rng = np.random.default_rng(10)
    xs = np.concatenate([rng.normal(size=(400, 4)) * 10.0 ** rng.integers(-6, 4, (400, 1)),
                         rng.normal(size=(100, 4)).astype(np.float16).astype(np.float64) * 300])
    for v in xs.astype(np.float32):
        want = R.exact_mul_f32(v[0], v[0])
        for m in (1, 2, 3):
            want = R.exact_fma_f32(v[m], v[m], want)
        got = O.norm2(v)
        assert got == want and got.tobytes() == want.tobytes(), v


def test_half_norm_code_matches_numpy():
    rng = np.random.default_rng(11)
    s2 = np.concatenate([np.abs(rng.normal(size=3000)).astype(np.float32) * np.float32(10.0) ** rng.integers(-12, 9, 3000).astype(np.float32),
                         np.float32([0.0, 1.0, 4.0, 9.0, 1e-30, 1.7e10])]).astype(np.float32)
    for v in s2:
        want = (np.sqrt(np.float32(v)) * np.float32(0.5)).astype(np.float16).view(np.uint16)
        assert O.half_norm_bits(v) == int(want), v


@pytest.mark.parametrize("S", [1, 3, 8, 32])
def test_nearest_matches_kdtree(S):
    rng = np.random.default_rng(100 + S)
    q = O.make_codebook(3, 1, 1, 0, S)[0, 0]
    cw = R.codewords_matrix_rep(q, np.array(R.hurwitz_units_in_oracle_order()))
    tree = cKDTree(cw)
    for _ in range(1500):
        x = rng.normal(size=4).astype(np.float32)
        k, gap = O.nearest(x, q)
        u = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64))
        _, kk = tree.query(u)
        scores = cw @ u
        top2 = np.sort(scores)[-2:]
        assert abs(gap - (top2[1] - top2[0])) < 1e-12
        if gap > 1e-9:
            assert k == kk
        else:
            assert scores[k] >= scores.max() - 1e-12


def test_codeword_inputs_map_to_themselves():
    rng = np.random.default_rng(12)
    q = O.make_codebook(0, 1, 1, 0, 32)[0, 0]
    for k in rng.integers(0, 24 * 32, 300):
        c = O.codeword(q, int(k))
        x = (c * rng.uniform(0.1, 100)).astype(np.float32)
        kk, gap = O.nearest(x, q)
        assert kk == k and gap > 1e-6


def test_deep_hole_six_way_tie_takes_smallest_code():
    """u = (1,1,0,0)/sqrt2 is a deep hole of the 24-cell: cos 45 degrees to 6
    vertices (+1, +i and the four (1,1,+-1,+-1)/2).  Ties keep the smallest k."""
    q = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    k, gap = O.nearest(np.float32([1, 1, 0, 0]), q)
    assert k == 0 and gap == 0.0
    u = np.array([1, 1, 0, 0]) / np.sqrt(2)
    t2 = O.t2_elements()
    assert int(np.sum(np.abs(t2 @ u - 1 / np.sqrt(2)) < 1e-12)) == 6
    # and the 24-cell's covering radius is 45 degrees: no direction is farther
    rng = np.random.default_rng(13)
    U = rng.normal(size=(20000, 4))
    U /= np.linalg.norm(U, axis=1, keepdims=True)
    assert (U @ t2.T).max(1).min() >= 1 / np.sqrt(2) - 1e-12


def test_s1_identity_codebook_is_nearest_24cell_vertex_closed_form():
    """With q_1 = 1 the codebook is 2T itself.  The best unit vertex scores
    max|u_m|, the best half vertex scores sum|u_m| / 2 (signs follow u)."""
    rng = np.random.default_rng(14)
    q = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    for _ in range(2000):
        x = rng.normal(size=4).astype(np.float32)
        k, gap = O.nearest(x, q)
        u = x / np.linalg.norm(x.astype(np.float64))
        a = np.abs(u)
        if gap < 1e-9:
            continue
        if a.max() >= a.sum() / 2:
            m = int(np.argmax(a))
            assert k == 2 * m + (1 if u[m] < 0 else 0)
        else:
            assert k == 8 + sum((1 << m) for m in range(4) if u[m] < 0)


def test_zero_chunk():
    r = O.encode_range(np.zeros((2, 8), np.float32), O.make_codebook(0, 1, 1, 0, 8)[0, 0])
    assert np.all(r["codes"] == 0) and np.all(r["hnorm"] == 0) and np.all(np.isinf(r["gap"]))
