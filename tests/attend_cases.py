"""Decode-step attention through the C ABI compared with the oracle.

The GPU encodes K and V, then ``hqmq_attend`` reads the records; the oracle
encodes the same input bytes itself, decodes them (rounded to binary16, the
values the decoder writes) and runs its plain attention per (sequence, KV
head) over the query heads of the group.  Records must agree except for
near-tie codes (two codewords within 1e-6, both correct); there the reference
decodes the GPU's choice, so the attention comparison tests the attention.

Tolerance, per output element of dimension d:

    |out - ref| <= 2^-9 * max_t |v[t][d]| + 2^-20 * max_{t,d'} |v[t][d']|

The first term bounds the weight rounding: each weight enters the value sum
rounded to binary16 (relative error <= 2^-11) and the normaliser sums the same
rounded weights, so the output moves by at most 2 * 2^-11 / (1 - 2^-11) times
max_t |v[t][d] - out[d]| <= 2 max_t |v[t][d]|.  The second covers fp32
accumulation of scores and sums (at most a few thousand terms per wave).
Decoded values agree exactly except where the decoder's fp32 product lands
within an fp32 rounding of a binary16 boundary (one binary16 ulp, rare); the
bound leaves room for that too.
"""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_quantization_hqmq_amd as K
import oracle as O
import synth
from tests import gpu_cases as GC
from tests import parity as P

WEIGHT_REL = 2.0 ** -9
ABS_REL = 2.0 ** -20


def f16_values(y64: np.ndarray) -> np.ndarray:
    return O.round_f16(y64).view(np.float16).astype(np.float64)


def oracle_slice(x: np.ndarray, q: np.ndarray, t0: int, B: int, C: float, npack: bool = False,
                 exact: bool = False):
    """Oracle records and binary16 decoded values of tokens [t0, t0+T) of one
    slice (t0 a multiple of the Med3x batch).  r["hrec"] is the norm record
    as the GPU stores it: binary16 codes, or (npack) compact codes, or
    (exact) exact-rate norm codes, whose half-norms the decode then uses."""
    T, D = x.shape
    r = O.encode_range(x, q, t0, B, C)
    hn = r["hnorm"]
    r["hrec"] = hn
    if exact:
        r["hrec"] = O.exact_norms(hn, q.shape[0])
        hn = O.exact_norm_to_h16(r["hrec"], q.shape[0])
    elif npack:
        b = O.code_bits(q.shape[0])
        r["hrec"] = O.compact_norms(hn, b)
        hn = O.compact_to_h16(r["hrec"], b)
    r["h16"] = hn
    return r, oracle_decode(r, r["codes"], q, T, D, t0, B)


def oracle_decode(r: dict, codes: np.ndarray, q: np.ndarray, T: int, D: int, t0: int, B: int) -> np.ndarray:
    """Binary16 values the oracle decodes from r's records with the given
    codes (the oracle's own, or the GPU's where they pick the other side of a
    near tie)."""
    y = O.decode_range(codes, r["h16"], T, D, q, r["side_pos"] if B else None,
                       r["side_val"] if B else None, t0)
    return f16_values(y)


def gpu_slice_records(desc: K.Desc, rec, l: int, h: int, t0: int, T: int):
    """GPU codes, hnorm and side entries of tokens [t0, t0+T) of slice (l, h)."""
    L, H, Tt, D = desc.shape
    cpt = D // 4
    b = O.code_bits(int(desc.S))
    if desc.norm_format == K.HQMQ_NORM_EXACT:
        assert t0 % 4 == 0
        words = rec.idx[l, h, t0 // 4:(t0 + T + 3) // 4].cpu().numpy().view(np.uint32)
        codes, hn = O.unpack_exact(words, T, cpt, int(desc.S))
        codes, hn = codes.reshape(-1), hn.reshape(-1)
    else:
        codes = P.unpack_words(rec.idx[l, h, t0:t0 + T].cpu().numpy().view(np.uint32), cpt, b).reshape(-1)
    if desc.norm_format == K.HQMQ_NORM_EXACT:
        pass
    elif desc.norm_format == K.HQMQ_NORM_PACKED:
        hn = P.unpack_words(rec.hnorm[l, h, t0:t0 + T].cpu().numpy().view(np.uint32), cpt, b).reshape(-1)
    else:
        hn = rec.hnorm[l, h, t0:t0 + T].cpu().numpy().view(np.uint16).reshape(-1)
    pos = val = None
    B = int(desc.med_batch_tokens)
    if B > 0:
        Bc = min(B, Tt)
        nb = (Tt + Bc - 1) // Bc
        offs = rec.batch_offsets.cpu().numpy().view(np.uint64)
        sl = l * H + h
        e0, e1 = int(offs[sl * nb + t0 // Bc]), int(offs[sl * nb + (t0 + T - 1) // Bc + 1])
        pos = rec.out_pos[e0:e1].cpu().numpy().view(np.uint32)
        val = rec.out_val[e0:e1].cpu().numpy().view(np.uint16)
    return codes, hn, pos, val


def record_mismatches(r: dict, g, mask: bool = False):
    """(codes that differ where the oracle's top-2 gap is below 1e-6 -- both
    choices are correct there --, every other difference); with mask, also
    the boolean mask of those near-tie codes."""
    codes, hn, pos, val = g
    diff = codes != r["codes"].reshape(-1)
    near = diff & (r["gap"].reshape(-1) < P.GAP_EXEMPT)
    bad = int((diff & ~near).sum()) + int((hn != r["hrec"].reshape(-1)).sum())
    if pos is not None:
        if len(pos) != len(r["side_pos"]):
            bad += abs(len(pos) - len(r["side_pos"])) + 1
        else:
            bad += int((pos != r["side_pos"]).sum()) + int((val != r["side_val"]).any(axis=1).sum())
    if mask:
        return int(near.sum()), bad, near
    return int(near.sum()), bad


def reference_slice(x: np.ndarray, q: np.ndarray, t0: int, B: int, C: float, desc: K.Desc, rec, l: int, h: int,
                    npack: bool = False, exact: bool = False):
    """Oracle records of tokens [t0, t0 + T) of slice (l, h) checked against
    the GPU's, and the decoded values the attention reference uses: the
    oracle's, except that where the GPU took the other side of a near tie
    (allowed) the oracle decodes the GPU's code.  Returns (values, near-tie
    codes, other record differences)."""
    T, D = x.shape
    r, dec = oracle_slice(x, q, t0, B, C, npack, exact)
    g = gpu_slice_records(desc, rec, l, h, t0, T)
    near, bad, near_mask = record_mismatches(r, g, mask=True)
    if near:
        codes = np.where(near_mask, g[0], r["codes"].reshape(-1)).reshape(r["codes"].shape)
        dec = oracle_decode(r, codes, q, T, D, t0, B)
    return dec, near, bad


def compare_out(got: np.ndarray, ref: np.ndarray, v: np.ndarray) -> float:
    """Largest error / tolerance over the group's outputs (0 when exact)."""
    if v.shape[0] == 0:
        return 0.0 if not np.any(got) else np.inf
    vmax = np.abs(v).max(axis=0)
    tol = WEIGHT_REL * vmax + ABS_REL * vmax.max() + 1e-30
    return float((np.abs(got - ref) / tol).max())


def make_queries(batch: int, hq: int, D: int, seed: int, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((batch, hq, D), generator=g, device=device).to(torch.float16)


def run_case(w: synth.Workload, seqs, group: int, scale: float, layers=None, max_len=None, seed=0,
             norm_format: int = K.HQMQ_NORM_F16, xform=None):
    """Encode w's K and V on the GPU, attend over seqs = [(start, len)], and
    compare every (layer, sequence, query head) with the oracle.  Returns a
    report with the worst error / tolerance ratio, the near-tie codes the two
    encoders chose differently (allowed) and every other record difference
    (must be 0).  xform(role, x), if given, changes the generated input of a
    role in place before both sides encode it."""
    desc = GC.desc_for(w, norm_format=norm_format)
    npack = norm_format == K.HQMQ_NORM_PACKED
    exact = norm_format == K.HQMQ_NORM_EXACT
    L, H, Tt, D = desc.shape
    xs, cbh, cbd, recs = {}, {}, {}, {}
    for role in (0, 1):
        xs[role] = synth.generate(w, role, "cuda")
        if xform is not None:
            xform(role, xs[role])
        cbh[role], cbd[role] = GC.codebook(w, role)
        recs[role] = K.encode(desc, xs[role], cbd[role])
    nb = len(seqs)
    starts = torch.tensor([s for s, _ in seqs], dtype=torch.int64, device="cuda")
    lens = torch.tensor([n for _, n in seqs], dtype=torch.int32, device="cuda")
    if max_len is None:
        max_len = max([n for _, n in seqs] + [0])
    q = make_queries(nb, H * group, D, seed)
    qn = q.float().cpu().numpy().astype(np.float64)
    rep = {"max_ratio": 0.0, "near_tie_codes": 0, "record_mismatch": 0, "outputs": 0}
    for l in (range(L) if layers is None else layers):
        out = K.attend(desc, l, recs[0], cbd[0], recs[1], cbd[1], q, starts, lens, max_len, scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for h in range(H):
            dec = {}
            for role in (0, 1):
                x = xs[role][l, h].float().cpu().numpy()
                dec[role], near, bad = reference_slice(x, cbh[role][l, h], 0, w.med_batch_tokens, w.med_C, desc,
                                                       recs[role], l, h, npack, exact)
                rep["near_tie_codes"] += near
                rep["record_mismatch"] += bad
            for b, (s, n) in enumerate(seqs):
                if s < 0 or s > Tt:
                    n_eff = 0
                else:
                    n_eff = max(0, min(n, max_len, Tt - s))
                kk, vv = dec[0][s:s + n_eff], dec[1][s:s + n_eff]
                ref = O.attend(kk, vv, qn[b, h * group:(h + 1) * group], scale)
                ratio = compare_out(got[b, h * group:(h + 1) * group], ref, vv)
                rep["max_ratio"] = max(rep["max_ratio"], ratio)
                rep["outputs"] += group * D
    return rep
