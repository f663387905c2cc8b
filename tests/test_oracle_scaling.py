"""Statistical check of the covering-rate claim (not a parity pin).

Proposition 3.1 (gist.science/nl technical summary, Methodologie 2): a random
multiplicative packing of 24 S codewords reaches covering rate
O((24 S)^(-1/3)) on S^3.  The constant is not given, so only the trend is
checked: the mean angular error at S = 32 over that at S = 8 should be near
4^(-1/3) = 0.63.  Parity of quality constants is unpinned.
"""
import numpy as np

import oracle as O


def _mean_angle(S, n=20000, seed=30):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(n // 32, 128)).astype(np.float32)
    q = O.make_codebook(11, 1, 1, 0, S)[0, 0]
    r = O.encode_range(x, q)
    cw = np.stack([O.codeword(q, k) for k in range(24 * S)])
    u = x.reshape(-1, 4).astype(np.float64)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    cos = np.einsum("ij,ij->i", u, cw[r["codes"]])
    return np.degrees(np.arccos(np.clip(cos, -1, 1))).mean()


def test_covering_rate_trend():
    a1, a8, a32 = _mean_angle(1), _mean_angle(8), _mean_angle(32)
    assert a1 > a8 > a32
    ratio = a32 / a8
    assert abs(ratio - 4 ** (-1 / 3)) < 0.06, (a8, a32, ratio)
