"""Pins of the oracle's binary16 conversion, its Philox4x64-10 generator and
the seeded codebook sampler.

binary16 is checked against numpy's float16 casts; Philox against
numpy.random.Philox (the same published generator, SC'11); the sampler's
output against the uniform law on S^3 (the pages: "random unit quaternions",
gist.science/nl technical summary, Methodologie 1 and 2).  The codebook's
concrete values are a reading of the pages (they name no generator).
"""
import numpy as np
import pytest
from scipy import stats

import oracle as O


def test_f16_value_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([O.f16_value(int(h)) for h in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros
    assert np.signbit(O.f16_value(0x8000)) and not np.signbit(O.f16_value(0))


def test_f16_bits_against_numpy():
    rng = np.random.default_rng(4)
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float64)
    finite.sort()
    mids = (finite[1:] + finite[:-1]) / 2          # exact ties
    near = np.concatenate([mids * (1 + 1e-12), mids * (1 - 1e-12)])
    rand = np.concatenate([rng.normal(size=20000) * 10.0 ** rng.integers(-9, 5, 20000),
                           [65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 2.0 ** -25,
                            2.0 ** -26, 3 * 2.0 ** -26, 1e-30, 0.0, -0.0]])
    with np.errstate(over="ignore"):
        for v in np.concatenate([finite, mids, near, rand]):
            want = int(np.array(v).astype(np.float16).view(np.uint16))
            assert O.f16_bits(v) == want, v


def test_round_f16_vectorised():
    y = np.random.default_rng(5).normal(size=1000) * 100
    np.testing.assert_array_equal(O.round_f16(y), y.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("key", [(0, 0), (5, 77), (2**64 - 1, 12345678901234567)])
@pytest.mark.parametrize("j", [0, 1, 2, 1000, 2**64 - 1])
def test_philox_matches_numpy(key, j):
    # numpy increments its 256-bit counter before producing each block
    c = (j - 1) % 2**256
    counter = np.array([(c >> (64 * w)) & (2**64 - 1) for w in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=counter)
    want = bg.random_raw(4)
    got = O.philox4x64_10([j % 2**64, 0 if j < 2**64 else 1, 0, 0], key)
    np.testing.assert_array_equal(got, want)


def test_codebook_unit_deterministic_and_keyed():
    a = O.make_codebook(0, 3, 4, 0, 32)
    b = O.make_codebook(0, 3, 4, 0, 32)
    np.testing.assert_array_equal(a, b)
    n = np.linalg.norm(a.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-6
    v = O.make_codebook(0, 3, 4, 1, 32)
    s1 = O.make_codebook(1, 3, 4, 0, 32)
    assert not np.any(np.all(a == v, axis=-1))
    assert not np.any(np.all(a == s1, axis=-1))
    # distinct (layer, head) slices differ
    flat = a.reshape(12, 32, 4)
    for i in range(12):
        for j in range(i + 1, 12):
            assert not np.array_equal(flat[i], flat[j])
    # the first S codewords do not depend on S
    np.testing.assert_array_equal(O.make_codebook(0, 3, 4, 0, 8), a[:, :, :8])


def test_codebook_is_uniform_on_s3():
    """Uniform on S^3: E q = 0, E q q^T = I/4, and each coordinate has the
    marginal density (2/pi) sqrt(1 - t^2)."""
    q = O.make_codebook(7, 1, 1, 0, 40000)[0, 0].astype(np.float64)
    N = len(q)
    assert np.abs(q.mean(0)).max() < 5 * 0.5 / np.sqrt(N)
    C = q.T @ q / N
    assert np.abs(C - np.eye(4) / 4).max() < 5 * 0.2 / np.sqrt(N)

    def cdf(t):
        t = np.clip(t, -1, 1)
        return 0.5 + (t * np.sqrt(1 - t * t) + np.arcsin(t)) / np.pi

    for m in range(4):
        assert stats.kstest(q[:, m], cdf).pvalue > 1e-4
    # pairs of coordinates are uncorrelated in sign (no axis preference)
    assert abs(np.mean(np.sign(q[:, 0] * q[:, 1]))) < 5 / np.sqrt(N)


def test_codebook_values_are_on_the_double_binary16_grid():
    """Codebook values are used as h + l, h = fp16(q), l = fp16(q - h)
    (numpy's float16 rounding here); generated codebooks are on that grid."""
    rng = np.random.default_rng(8)
    qs = np.concatenate([rng.uniform(-1, 1, 5000), rng.normal(size=2000) * 1e-3,
                         [1.0, -1.0, 0.0, 1e-6, -3e-5, 0.999999]]).astype(np.float32)
    for q in qs:
        h = np.float16(q)
        l = np.float16(np.float32(q) - np.float32(h))
        assert O.codebook_value(q) == float(h) + float(l), q
    cb = O.make_codebook(3, 2, 3, 1, 64).ravel()
    assert all(O.codebook_value(v) == float(v) for v in cb)
    # 22 significant bits: within 2^-22 of the fp32 value for normal-range parts
    q = rng.uniform(0.25, 1, 1000).astype(np.float32)
    err = np.array([abs(O.codebook_value(v) - float(v)) / float(v) for v in q])
    assert err.max() <= 2.0 ** -22
