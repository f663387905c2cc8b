"""Pins of the oracle's Med3x step, record packing, decoding and byte
accounting.

Med3x (gist.science/nl technical summary, Methodologie 3; the abstract):
the median chunk norm of the batch, chunks with r > C r_med (C = 3) kept in
fp16 with a one-bit flag, the rest quantised.  The pins: numpy's partition
for the median, designed batches whose outlier set is known, the strict '>'
boundary, the floor(n/2) bound.  Decoding is pinned by its closed form, the
packing by an independent bit-level unpack, the byte accounting by the
pages' "43 GB" for the Llama-3-70B 128k cache.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth
from tests import refmath as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
C3 = float(GOLD["med3_C"]["value"])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 64, 1000, 1001])
def test_lower_median_matches_partition(n):
    rng = np.random.default_rng(n)
    for trial in range(5):
        keys = (rng.integers(0, 6, n) if trial % 2 else rng.exponential(size=n)).astype(np.float32)
        want = np.partition(keys, (n - 1) // 2)[(n - 1) // 2]
        assert O.lower_median(keys) == want


def test_threshold_is_fp32_c2_times_median():
    rng = np.random.default_rng(20)
    for med in np.abs(rng.normal(size=500)).astype(np.float32) * np.float32(7.3):
        assert O.med3_threshold(med, C3) == np.float32(np.float32(C3) * np.float32(C3)) * med


def _chunks(norms):
    """One chunk per norm, along the real axis: (r, 0, 0, 0)."""
    x = np.zeros((len(norms), 4), np.float32)
    x[:, 0] = norms
    return x.reshape(-1, 4)


def _encode_chunks(x, q, B_chunks):
    """Encode a flat chunk list as a slice with one chunk per token (D = 4)."""
    return O.encode_range(x.reshape(-1, 4), q, 0, B_chunks, C3)


def test_designed_batch_exact_outliers():
    rng = np.random.default_rng(21)
    q = O.make_codebook(0, 1, 1, 0, 8)[0, 0]
    n, m = 1000, 37
    norms = np.ones(n, np.float32)
    # 2.5 r_med is not an outlier with C = 3 (it would be with C in place of C^2)
    norms[rng.choice(n, 100, replace=False)] = 2.5
    out_idx = np.sort(rng.choice(np.where(norms == 1)[0], m, replace=False))
    norms[out_idx] = 10.0
    r = _encode_chunks(_chunks(norms), q, n)
    assert list(r["side_pos"]) == list(out_idx)
    assert list(r["batch_counts"]) == [m]
    assert np.all((r["hnorm"] & 0x8000 != 0) == (norms == 10.0))
    # side values are the fp16 values of the chunk
    np.testing.assert_array_equal(r["side_val"][:, 0], np.float16(10.0).view(np.uint16))
    # flagged records keep their half-norm in the low 15 bits
    assert np.all((r["hnorm"][out_idx] & 0x7FFF) == np.float16(5.0).view(np.uint16))


def test_strict_greater_boundary():
    """r exactly C r_med is bulk; just above it is an outlier."""
    q = O.make_codebook(0, 1, 1, 0, 8)[0, 0]
    norms = np.float32([1, 1, 1, 1, 1, 3.0, np.nextafter(np.float32(3.0), np.float32(10))])
    r = _encode_chunks(_chunks(norms), q, len(norms))
    assert list(r["side_pos"]) == [6]


def test_floor_half_bound_and_zero_median():
    rng = np.random.default_rng(22)
    q = O.make_codebook(0, 1, 1, 0, 8)[0, 0]
    for n in (2, 3, 10, 11, 257):
        # more than half zeros: median 0, every nonzero chunk is an outlier
        norms = np.zeros(n, np.float32)
        nz = rng.choice(n, n // 2, replace=False)
        norms[nz] = rng.uniform(0.5, 2.0, len(nz))
        r = _encode_chunks(_chunks(norms), q, n)
        assert len(r["side_pos"]) == len(nz) <= n // 2
        # adversarial spread: never more than floor(n/2) outliers
        norms = np.exp(rng.normal(size=n) * 5).astype(np.float32)
        r = _encode_chunks(_chunks(norms), q, n)
        assert len(r["side_pos"]) <= n // 2


def test_batches_and_partial_tail():
    rng = np.random.default_rng(23)
    q = O.make_codebook(0, 1, 1, 0, 8)[0, 0]
    T, D, B = 70, 16, 32            # batches of 32, 32 and a partial 6 tokens
    x = rng.normal(size=(T, D)).astype(np.float32)
    x[5, 4:8] *= 40
    x[40, 0:4] *= 40
    x[68, 12:16] *= 40
    r = O.encode_range(x, q, 0, B, C3)
    cpt = D // 4
    s2 = r["s2"]
    want = []
    for b in range(3):
        lo, hi = b * B * cpt, min((b + 1) * B, T) * cpt
        med = np.partition(s2[lo:hi], (hi - lo - 1) // 2)[(hi - lo - 1) // 2]
        thr = np.float32(9.0) * med
        want.append(int((s2[lo:hi] > thr).sum()))
        assert r["batch_counts"][b] == want[-1]
    assert {5 * cpt + 1, 40 * cpt + 0, 68 * cpt + 3} <= set(r["side_pos"].tolist())
    assert np.all(np.diff(r["side_pos"].astype(np.int64)) > 0)
    # a token offset shifts the stored positions
    r2 = O.encode_range(x[32:], q, 32, B, C3)
    np.testing.assert_array_equal(r2["side_pos"], r["side_pos"][r["side_pos"] >= 32 * cpt])


@pytest.mark.parametrize("S,D", [(1, 16), (8, 128), (11, 64), (32, 128), (1024, 32)])
def test_pack_row_bit_layout(S, D):
    b = O.code_bits(S)
    assert 2 ** b >= 24 * S > 2 ** (b - 1)
    cpt = D // 4
    W = O.words_per_row(S, D)
    rng = np.random.default_rng(S)
    codes = rng.integers(0, 24 * S, cpt).astype(np.int32)
    words = O.pack_row(codes, b, W)
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    got = [int(sum(int(bits[c * b + i]) << i for i in range(b))) for c in range(cpt)]
    assert got == codes.tolist()
    assert not bits[cpt * b:].any()
    np.testing.assert_array_equal(O.unpack_row(words, cpt, b), codes)


def test_code_width_for_quoted_codebooks():
    """192 codewords need 8 bits, 768 need 10.  The pages' 3.79 bits at S=8 is
    log2(192)/2 (their rate; the stored format here is a reading)."""
    assert O.code_bits(8) == 8 and O.code_bits(32) == 10
    assert abs(math.log2(192) / 2 - GOLD["bits_quoted"]["value"]["8"]) < 0.005


def test_decode_closed_form_and_round_trip():
    rng = np.random.default_rng(24)
    S, D, T = 32, 16, 50
    q = O.make_codebook(0, 1, 1, 0, S)[0, 0]
    cw = R.codewords_matrix_rep(q, np.array(R.hurwitz_units_in_oracle_order()))
    # decode of arbitrary records: y = 2 h c_k
    codes = rng.integers(0, 24 * S, T * D // 4).astype(np.int32)
    hn = np.abs(rng.normal(size=T * D // 4)).astype(np.float16).view(np.uint16)
    y = O.decode_range(codes, hn, T, D, q)
    want = 2.0 * hn.view(np.float16).astype(np.float64)[:, None] * cw[codes]
    np.testing.assert_allclose(y.reshape(-1, 4), want, rtol=0, atol=1e-12)
    # round trip of codeword inputs rho c_k: exact code, value within the
    # binary16 rounding of the norm
    ks = rng.integers(0, 24 * S, T * D // 4)
    rho = rng.uniform(0.5, 20, len(ks))
    x = (rho[:, None] * cw[ks]).astype(np.float32).reshape(T, D)
    r = O.encode_range(x, q)
    assert np.array_equal(r["codes"], ks)
    y = O.decode_range(r["codes"], r["hnorm"], T, D, q).reshape(-1, 4)
    assert np.abs(y - x.reshape(-1, 4)).max() <= 2.0 ** -10 * rho.max()


def test_outlier_values_round_trip_exactly():
    rng = np.random.default_rng(25)
    q = O.make_codebook(0, 1, 1, 0, 8)[0, 0]
    x = rng.normal(size=(64, 32))
    x[3] *= 200
    x = x.astype(np.float16).astype(np.float32)
    r = O.encode_range(x, q, 0, 64, C3)
    assert len(r["side_pos"]) > 0
    y = O.decode_range(r["codes"], r["hnorm"], 64, 32, q, r["side_pos"], r["side_val"])
    for p in r["side_pos"]:
        t, c = divmod(int(p), 8)
        np.testing.assert_array_equal(y[t, 4 * c:4 * c + 4], x[t, 4 * c:4 * c + 4])


def test_fp16_cache_bytes_of_the_pages_example():
    """80 layers x 8 KV heads x 131072 tokens x 128 x K,V x 2 B = 42.95e9 B:
    the pages' "43 GB" Llama-3-70B 128k cache."""
    w = synth.WORKLOADS[4]
    b = synth.fp16_bytes(w)
    assert b == 42_949_672_960
    assert round(b / 1e9) == GOLD["llama3_70b_128k_fp16_cache_GB"]["value"]


def test_tensor_helpers_round_trip():
    rng = np.random.default_rng(26)
    L, H, T, D, S, B = 2, 3, 40, 32, 8, 16
    x = rng.normal(size=(L, H, T, D)).astype(np.float32)
    x[1, 2, 7, 4:8] = 300
    cb = O.make_codebook(0, L, H, 0, S)
    enc = O.encode_tensor(x, cb, B, C3)
    nb = (T + B - 1) // B
    assert len(enc["batch_offsets"]) == L * H * nb + 1
    assert enc["batch_offsets"][-1] == len(enc["side_pos"]) >= 1
    y = O.decode_tensor(enc, cb, x.shape, B)
    flagged = (enc["hnorm"] & 0x8000) != 0
    r = 2.0 * (enc["hnorm"] & 0x7FFF).view(np.float16).astype(np.float64)
    err = np.abs(y - x).reshape(L, H, T, D // 4, 4).max(-1)
    assert np.all(err[flagged] == 0)
    # bulk error is bounded by the chord to the chosen codeword (<= r)
    assert np.all(err[~flagged] <= 1.2 * r[~flagged] + 1e-6)
