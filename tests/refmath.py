"""Independent textbook mathematics used to pin the oracle.

Nothing here is copied from the oracle: quaternions are multiplied through
their 2x2 complex-matrix representation, the unit Hurwitz quaternions are
enumerated from their definition, fp32 rounding is done on exact rationals.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np


def qmat(q) -> np.ndarray:
    """2x2 complex matrix of q = a + b i + c j + d k (an algebra isomorphism
    of the quaternions onto a subalgebra of M2(C))."""
    a, b, c, d = (complex(v) for v in q)
    return np.array([[a + b * 1j, c + d * 1j], [-c + d * 1j, a - b * 1j]], dtype=np.complex128)


def qmat_inv(m: np.ndarray) -> np.ndarray:
    return np.array([m[0, 0].real, m[0, 0].imag, m[0, 1].real, m[0, 1].imag])


def qprod(a, b) -> np.ndarray:
    """Quaternion product through the matrix representation."""
    return qmat_inv(qmat(a) @ qmat(b))


def conj(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    return np.array([q[0], -q[1], -q[2], -q[3]])


def hurwitz_units() -> list:
    """All unit quaternions whose coordinates are all integers or all halves of
    odd integers (the unit group of the Hurwitz order)."""
    out = []
    vals = [-1.0, -0.5, 0.0, 0.5, 1.0]
    for v in itertools.product(vals, repeat=4):
        if abs(sum(x * x for x in v) - 1.0) > 1e-12:
            continue
        ints = all(float(x).is_integer() for x in v)
        halves = all(abs(x) == 0.5 for x in v)
        if ints or halves:
            out.append(tuple(v))
    return out


def codewords_matrix_rep(q: np.ndarray, t2: np.ndarray) -> np.ndarray:
    """All 24 S products t2[p] * q[s], index 24 s + p, via qprod."""
    S = q.shape[0]
    cw = np.zeros((24 * S, 4))
    for s in range(S):
        for p in range(24):
            cw[24 * s + p] = qprod(t2[p], q[s].astype(np.float64))
    return cw


def round_fraction_to_f32(r: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 of an exact rational."""
    if r == 0:
        return np.float32(0.0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e_q = max(e, -126) - 23           # quantum exponent (subnormals: 2^-149)
    scaled = a / (Fraction(2) ** e_q)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** e_q))


def exact_fma_f32(a: np.float32, b: np.float32, c: np.float32) -> np.float32:
    return round_fraction_to_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def exact_mul_f32(a: np.float32, b: np.float32) -> np.float32:
    return round_fraction_to_f32(Fraction(float(a)) * Fraction(float(b)))


def hurwitz_units_in_oracle_order() -> list:
    """2T in the order the codec indexes it (a reading, the pages give only the
    set): +1, -1, +i, -i, +j, -j, +k, -k, then (s0, s1, s2, s3)/2 with
    s_m = -1 exactly when bit m of (p - 8) is set."""
    out = []
    for p in range(8):
        v = [0.0] * 4
        v[p // 2] = 1.0 if p % 2 == 0 else -1.0
        out.append(v)
    for p in range(8, 24):
        out.append([-0.5 if ((p - 8) >> m) & 1 else 0.5 for m in range(4)])
    assert {tuple(v) for v in out} == set(hurwitz_units())
    return out
