"""GPU parity of the exact-rate records (HQMQ_NORM_EXACT) against the
oracle, through the C ABI.

Every chunk of small ragged shapes: token counts that end inside a group of 4
rows, every head_dim, S from 1 to 1024 (the codeword-table and the
per-chunk codeword decode paths), fp16 and fp32 inputs, Med3x on and off
(single- and two-pass select).  The bar (tests/parity.py): every norm code
bit-exact, every group word bit-exact where the group's index codes match the
oracle's (near ties aside), decoded values within 1e-3 of the chunk norm.
"""
import numpy as np
import pytest
import torch

import kv_cache_quantization_hqmq_amd as K
import oracle as O
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu


def _x(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda") * scale
    return x.clamp(-65504, 65504).to(dtype)


def _cb(L, H, S, role=0, seed=0):
    host = K.hqmq_make_codebook(seed, L, H, role, S)
    return host, torch.from_numpy(host).cuda()


def _check(desc, x, cb_host, cb_dev, capacity=None):
    print(f"case {tuple(desc.shape)} S={desc.S} dtype={desc.dtype} B={desc.med_batch_tokens} exact", flush=True)
    rec, y = G.run(desc, x, cb_dev, capacity)
    sz = K.hqmq_sizes(desc)
    assert rec.idx.numel() * 4 == sz.idx_bytes and sz.hnorm_bytes == 0
    rep = G.compare(desc, x, cb_host, rec, y)
    print(dict(rep), flush=True)
    return rep, rec, y


CASES = [
    # (layers, heads, tokens, head_dim, S, dtype, med_batch_tokens)
    (2, 3, 1001, 128, 8, "f16", 0),
    (2, 3, 1501, 128, 32, "f16", 512),
    (1, 2, 777, 64, 16, "f16", 256),
    (1, 2, 333, 256, 1, "f32", 100),
    (2, 1, 130, 16, 2, "f16", 64),
    (1, 3, 65, 32, 64, "f32", 0),
    (1, 1, 97, 128, 1024, "f16", 32),
    (1, 1, 4100, 128, 32, "f32", 4096),
    (3, 2, 2051, 128, 8, "f16", 1024),
    # batches above 131072 chunks take the two-pass Med3x select
    (1, 1, 4200, 256, 32, "f16", 2100),
]


@pytest.mark.parametrize("L,H,T,D,S,dt,B", CASES)
def test_exact_records_every_chunk(L, H, T, D, S, dt, B):
    dtype = torch.float16 if dt == "f16" else torch.float32
    x = _x((L, H, T, D), dtype, seed=L * 1000 + T + S + 7)
    if B > 0:
        x[:, :, :, 5] *= 40
        x[:, :, ::97, :] *= 9
    cb_host, cb = _cb(L, H, S)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F32 if dt == "f32" else K.HQMQ_F16, B, 3.0, K.HQMQ_NORM_EXACT)
    rep, _, _ = _check(desc, x, cb_host, cb)
    if B > 0:
        assert rep["outliers"] > 0


@pytest.mark.parametrize("S", [1, 8, 32])
def test_exact_norm_codes_of_every_binary16_half_norm(S):
    """Chunks (v, v, v, v) have half-norm exactly v (s2 = 4 v^2 exact, root
    2|v|): one chunk per finite non-negative binary16 value, so the GPU's
    exact-rate norm code is checked against the oracle's nearest-level search
    at every input pattern, including subnormals, level midpoints (ties to the
    even level) and values above the top level (the cap)."""
    v = np.arange(0x7C00, dtype=np.uint16).view(np.float16)
    cpt = 32
    T = -(-len(v) // cpt)
    vals = np.zeros(T * cpt, np.float16)
    vals[:len(v)] = v
    x = np.repeat(vals[:, None], 4, axis=1).reshape(1, 1, T, 4 * cpt)
    xt = torch.from_numpy(x).cuda()
    cb_host, cb = _cb(1, 1, S)
    desc = K.Desc.make(1, 1, T, 4 * cpt, S, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_EXACT)
    rep, rec, _ = _check(desc, xt, cb_host, cb)
    # the norm codes cover every finite level
    _, nc = O.unpack_exact(rec.idx[0, 0].cpu().numpy().view(np.uint32), T, cpt, S)
    levels = np.unique(nc)
    assert levels[0] == 0 and len(levels) >= min(24 * S - 2, 3000) * 0.95


def test_exact_decode_matches_the_f16_path_up_to_the_norm_code():
    """The exact and binary16 formats share the search: the same input gives
    the same index codes and outliers, and the exact decode equals the
    binary16 decode with each half-norm replaced by its level's value."""
    L, H, T, D, S = 1, 2, 1000, 128, 32
    x = _x((L, H, T, D), torch.float16, seed=3)
    x[:, :, :, 11] *= 50
    cb_host, cb = _cb(L, H, S)
    d16 = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, 256, 3.0, K.HQMQ_NORM_F16)
    dex = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, 256, 3.0, K.HQMQ_NORM_EXACT)
    r16, _ = G.run(d16, x, cb)
    rex, yex = G.run(dex, x, cb)
    assert r16.n_outliers == rex.n_outliers > 0
    assert torch.equal(r16.out_pos[:r16.n_outliers], rex.out_pos[:rex.n_outliers])
    assert torch.equal(r16.out_val[:r16.n_outliers], rex.out_val[:rex.n_outliers])
    cpt = D // 4
    for l in range(L):
        for h in range(H):
            codes_ex, _ = O.unpack_exact(rex.idx[l, h].cpu().numpy().view(np.uint32), T, cpt, S)
            from tests import parity as P
            codes_16 = P.unpack_words(r16.idx[l, h].cpu().numpy().view(np.uint32), cpt, O.code_bits(S))
            np.testing.assert_array_equal(codes_ex, codes_16)
