"""Pins of the oracle's exact-rate record (norm code with 24 S levels and
the mixed-radix group packing), CPU only.

The pages give the rate, not the format: about 3.79 bits per element at
S = 8 and about 5 at S = 32 (signal-ia-rouge.vercel.app, "La mecanique";
the abstract), i.e. two codes of log2(24 S) bits per 4-element chunk.  The
oracle's reading: a norm code with 24 S levels beside the 24 S-valued
index, each split into m plain bits and one ternary digit (24 S = 3 2^m),
digits packed eight to a 13-bit field, groups of 4 token rows.  These tests check
the oracle against things written independently of it: the defining
property of a nearest-level quantiser (a vectorised search over every
binary16 input), closed forms of the level grid, an unpacker written with
numpy's bit unpacking and integer base-3 digits, and the information
bound against the pages' quoted rates.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
POW2_S = (1, 2, 4, 8, 16, 32, 64, 256, 1024)


def _f16_values(patterns):
    return np.asarray(patterns, np.uint16).view(np.float16).astype(np.float64)


def _levels(S):
    """Finite levels of the oracle's grid (the grid itself is pinned below)."""
    R = 24 * S
    pats = []
    for n in range(R - 1):
        p = O.exact_level_pattern(n, S)
        if p >= 0x7C00:
            break
        pats.append(p)
    return np.array(pats, np.int64)


def test_m_splits_the_codeword_count():
    for S in POW2_S:
        m = O.exact_m(S)
        assert 24 * S == 3 * 2 ** m
    for S in (3, 5, 13, 100, 1000, 2048):
        assert O.exact_m(S) == -1


@pytest.mark.parametrize("S", POW2_S)
def test_level_grid_divides_the_binades_evenly(S):
    """R / 32 levels per binade of the binary16 pattern range: binade
    boundaries (patterns 1024 e) are levels whenever R / 32 is an integer,
    consecutive patterns are 32768 / R apart up to rounding, and the
    patterns increase strictly."""
    R = 24 * S
    pats = _levels(S)
    d = np.diff(pats)
    assert np.all(d > 0)
    step = 32768 / R
    assert np.all(np.abs(d - step) <= 1.0)
    # the level of pattern n: within half a pattern of n 32768 / R
    n = np.arange(len(pats))
    assert np.all(np.abs(pats - n * step) <= 0.5)
    if R % 32 == 0:
        L = R // 32
        for e in range(31):
            assert pats[e * L] == 1024 * e
    assert pats[-1] < 0x7C00 and (len(pats) == R - 1 or O.exact_level_pattern(len(pats), S) >= 0x7C00)


@pytest.mark.parametrize("S", (1, 2, 8, 32, 1024))
def test_exact_norm_is_the_nearest_level_for_every_binary16_input(S):
    """For every finite non-negative binary16 half-norm: the code is the level
    with the nearest value (a tie to the even level), found here by a
    vectorised search over all levels; flagged records give R - 1."""
    R = 24 * S
    pats = _levels(S)
    lv = _f16_values(pats)
    h = np.arange(0x7C00, dtype=np.uint16)
    hv = _f16_values(h)
    # nearest level: the insertion point and its left neighbour
    hi = np.clip(np.searchsorted(lv, hv, side="left"), 0, len(lv) - 1)
    lo = np.clip(hi - 1, 0, len(lv) - 1)
    dlo, dhi = np.abs(hv - lv[lo]), np.abs(lv[hi] - hv)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    got = O.exact_norms(h, S)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"S={S}: h={h[bad[0]]:#x} got {got[bad[0]]} want {want[bad[0]]}"
    # flags, including a flag over a nonzero pattern
    assert np.all(O.exact_norms(np.array([0x8000, 0xBC00, 0xFBFF], np.uint16), S) == R - 1)
    # and the code stands for that level's pattern
    back = O.exact_norm_to_h16(got[::97], S)
    assert np.array_equal(back, pats[got[::97]].astype(np.uint16))
    assert O.exact_norm_to_h16(np.array([R - 1]), S)[0] == 0x8000


@pytest.mark.parametrize("S", (8, 32))
def test_exact_norm_relative_error_bound(S):
    """Relative error of the decoded half-norm at most half a level step,
    (2^(32 / R) - 1) / 2 relative, over the normal range below the top level."""
    R = 24 * S
    pats = _levels(S)
    h = np.arange(0x0400, pats[-1], 7, dtype=np.uint16)
    v = _f16_values(h)
    dec = _f16_values(O.exact_norm_to_h16(O.exact_norms(h, S), S))
    rel = np.abs(dec - v) / v
    # pattern steps are 32768 / R (+-1): within a binade the value step is at
    # most (32768 / R + 1) / 1024 of the binade's start
    bound = 0.5 * (32768 / R + 1) / 1024
    assert rel.max() <= bound
    assert rel.max() > 0.5 * bound   # and not trivially finer


def _unpack_independent(words, T, cpt, S):
    """An unpacker written from the layout description only: numpy bit
    unpacking for the plain parts and the 13-bit digit fields, integer
    base-3 digits of each field."""
    m = int(round(math.log2(24 * S / 3)))
    wl = -(-cpt * m // 32)
    fh = -(-cpt // 8)
    codes = np.zeros((T, cpt), np.int64)
    norms = np.zeros((T, cpt), np.int64)
    for g in range(words.shape[0]):
        w = np.ascontiguousarray(words[g], np.uint32)
        dbits = np.unpackbits(w[8 * wl:].view(np.uint8), bitorder="little").astype(np.int64)
        fields = dbits[:4 * 2 * fh * 13].reshape(4, 2, fh, 13) @ (1 << np.arange(13))
        for r in range(min(4, T - 4 * g)):
            for plane, out in ((0, codes), (1, norms)):
                stream = np.unpackbits(w[(plane * 4 + r) * wl:(plane * 4 + r + 1) * wl].view(np.uint8),
                                       bitorder="little")
                lows = stream[:cpt * m].reshape(cpt, m).astype(np.int64) @ (1 << np.arange(m))
                for f in range(fh):
                    v = int(fields[r, plane, f])
                    assert v < 3 ** 8
                    for i in range(8):
                        v, d = divmod(v, 3)
                        if 8 * f + i < cpt:
                            out[4 * g + r, 8 * f + i] = d * 2 ** m + lows[8 * f + i]
                        else:
                            assert d == 0
    return codes, norms


@pytest.mark.parametrize("S,cpt,T", [(8, 32, 9), (32, 32, 4), (1, 4, 3), (2, 16, 5), (1024, 64, 6),
                                     (4, 8, 1), (64, 32, 13)])
def test_pack_exact_round_trips_through_an_independent_unpacker(S, cpt, T):
    R = 24 * S
    rng = np.random.default_rng(S * 131 + cpt + T)
    codes = rng.integers(0, R, (T, cpt))
    norms = rng.integers(0, R, (T, cpt))
    # extremes in the first row: all zero and all R - 1
    codes[0, : cpt // 2] = R - 1
    norms[0, cpt // 2:] = R - 1
    words = O.pack_exact(codes, norms, S)
    assert words.shape == (-(-T // 4), O.exact_group_words(cpt, S))
    c2, n2 = _unpack_independent(words, T, cpt, S)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(n2, norms)
    c3, n3 = O.unpack_exact(words, T, cpt, S)
    np.testing.assert_array_equal(c3, codes)
    np.testing.assert_array_equal(n3, norms)
    # rows past T in the last group are zero
    if T % 4:
        zero = O.pack_exact(np.zeros((4 - T % 4, cpt), np.int64), np.zeros((4 - T % 4, cpt), np.int64), S)
        assert not zero.any()


def test_pack_exact_is_injective_on_single_changes():
    """Changing any one code or norm of a group changes its words."""
    S, cpt = 8, 32
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 192, (4, cpt))
    norms = rng.integers(0, 192, (4, cpt))
    base = O.pack_exact(codes, norms, S)
    for _ in range(200):
        r, c, which = int(rng.integers(4)), int(rng.integers(cpt)), int(rng.integers(2))
        a = (codes if which == 0 else norms).copy()
        a[r, c] = (a[r, c] + int(rng.integers(1, 192))) % 192
        w = O.pack_exact(a if which == 0 else codes, norms if which == 0 else a, S)
        assert not np.array_equal(w, base)


@pytest.mark.parametrize("S", POW2_S)
@pytest.mark.parametrize("cpt", (4, 16, 32, 64))
def test_group_size_against_the_information_bound(S, cpt):
    """A group of 4 rows holds 8 cpt values of log2(24 S) bits each: its
    size can not be smaller, and the packing loses little (digits at 13 / 8
    bits instead of log2 3, fields of 8 digits, and word padding)."""
    bits = 32 * O.exact_group_words(cpt, S)
    info = 8 * cpt * math.log2(24 * S)
    assert bits >= info
    m = O.exact_m(S)
    fields = 8 * -(-cpt // 8)
    assert bits <= 8 * cpt * m + fields * 13 + 8 * 31 + 31


def test_rates_at_the_pages_settings():
    """head_dim 128: 3.8125 bits per element at S = 8 and 4.8125 at S = 32,
    against the pages' two codes of log2(24 S) bits per chunk (3.79 and
    4.79, quoted as ~3.79 and ~5)."""
    q = GOLDEN["bits_quoted"]["value"]
    for S, want in ((8, 3.8125), (32, 4.8125)):
        per_elem = 32 * O.exact_group_words(32, S) / (4 * 128)
        assert per_elem == want
        exact = 2 * math.log2(24 * S) / 4
        assert exact <= per_elem <= exact * 1.006
        assert abs(per_elem - q[str(S)]) / q[str(S)] < 0.05
    assert round(2 * math.log2(24 * 8) / 4, 2) == q["8"]
