"""Pins of the compact norm code (the reading that gives the norm as many
bits b as the direction code, matching the pages' ~3.79 / ~5 bits per
element at S = 8 / 32: the binary16 half-norm rounded, ties to even, to a
float with 5 exponent bits and b - 5 mantissa bits).

The oracle's rounding is checked against a brute-force nearest-value search
over the whole format (every finite value enumerated from its bit pattern),
for every binary16 input; plus the identity at b = 15, monotonicity, the
relative error bound, the largest finite value and the outlier code.
CPU only."""
import numpy as np
import pytest

import oracle as O

ALL_H16 = np.arange(0x7C00, dtype=np.uint16)   # every finite non-negative binary16


def _format_values(b):
    """All finite values of the format, in code order (code c <-> binary16
    pattern c << (15 - b)), excluding the all-ones (outlier) code and the
    infinities of exponent 31."""
    m = b - 5
    codes = np.arange((31 << m), dtype=np.uint32)
    return codes, (codes << (15 - b)).astype(np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("b", [5, 8, 9, 10, 12])
def test_rounds_to_the_nearest_value_ties_to_even(b):
    codes, vals = _format_values(b)
    got = O.compact_norms(ALL_H16, b)
    x = ALL_H16.view(np.float16).astype(np.float64)
    # brute force: nearest format value; exact ties take the even code
    for lo in range(0, len(x), 4096):
        xs = x[lo:lo + 4096, None]
        d = np.abs(vals[None, :] - xs)
        dmin = d.min(axis=1, keepdims=True)
        cand = np.where(d == dmin, codes[None, :], np.uint32(0xFFFFFFFF))
        even = np.where((cand & 1) == 0, cand, np.uint32(0xFFFFFFFF)).min(axis=1)
        any_ = cand.min(axis=1)
        ntie = (d == dmin).sum(axis=1)
        want = np.where(ntie > 1, even, any_)
        np.testing.assert_array_equal(got[lo:lo + 4096], want)


def test_full_width_is_the_identity():
    np.testing.assert_array_equal(O.compact_norms(ALL_H16, 15), ALL_H16.astype(np.uint32))


@pytest.mark.parametrize("b", [5, 8, 10, 13])
def test_monotone_bounded_and_flagged(b):
    m = b - 5
    got = O.compact_norms(ALL_H16, b)
    assert np.all(np.diff(got.astype(np.int64)) >= 0)
    assert got.max() == (31 << m) - 1            # the largest finite value caps
    assert O.compact_norms(np.array([0x8000, 0x8000 | 0x3C00], np.uint16), b).tolist() == [(1 << b) - 1] * 2
    # relative error of normal values at most half a unit in the last place
    x = ALL_H16.view(np.float16).astype(np.float64)
    y = (got << (15 - b)).astype(np.uint16).view(np.float16).astype(np.float64)
    normal = (x >= 2.0 ** -14) & (x <= (2 - 2.0 ** -m) * 2 ** 15)
    assert np.all(np.abs(y[normal] - x[normal]) <= x[normal] * 2.0 ** -(m + 1) + 1e-300)


def test_back_to_half_norm_records():
    assert O.compact_to_h16(np.array([(1 << 10) - 1]), 10).tolist() == [0x8000]
    np.testing.assert_array_equal(O.compact_to_h16(np.array([0, 480, 991]), 10),
                                  np.array([0, 480 << 5, 991 << 5], np.uint16))
