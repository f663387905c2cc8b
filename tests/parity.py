"""Parity comparison between the HIP path and the oracle (shared by the GPU
tests, the smoke check and the benchmark's sampled parity).

The bar (from the method's definition and the build's contract):
  * half-norm codes, Med3x flags, side-list positions/values and batch
    offsets: bit-exact;
  * codeword indices: exact wherever the oracle's top-2 score gap is at least
    1e-6; below that several codes are correct, and the GPU's choice must
    score within 1e-6 of the oracle's best;
  * packed index words: bit-exact on every token row whose codes all match;
  * packed norm format: the compact norm codes, and so their words, bit-exact
    (they follow from the half-norm codes, which are exact);
  * exact-rate format: every norm code bit-exact, every group word bit-exact
    in groups whose index codes all match;
  * decoded values: |y_gpu - y_oracle| <= 1e-3 * r^ per element (r^ the
    decoded chunk norm), outlier chunks exact.
"""
from __future__ import annotations

import numpy as np

import oracle as O
from tests import refmath as R

GAP_EXEMPT = 1e-6
REL_TOL = 1e-3


def unpack_words(words: np.ndarray, cpt: int, b: int) -> np.ndarray:
    """[..., W] u32 rows -> [..., cpt] codes (independent numpy unpacker)."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    lead = w.shape[:-1]
    bits = np.unpackbits(w.reshape(-1, w.shape[-1]).view(np.uint8), axis=1, bitorder="little")
    bits = bits[:, :cpt * b].reshape(-1, cpt, b).astype(np.int64)
    codes = bits @ (np.int64(1) << np.arange(b, dtype=np.int64))
    return codes.reshape(*lead, cpt)


def codeword_table(q: np.ndarray) -> np.ndarray:
    """All 24 S codewords of one slice, k = 24 s + p, via the matrix
    representation (independent of both the oracle and the kernels)."""
    return R.codewords_matrix_rep(np.asarray(q, np.float32), np.array(R.hurwitz_units_in_oracle_order()))


class Report(dict):
    def merge(self, other: dict):
        for k, v in other.items():
            if isinstance(v, (int, np.integer)):
                self[k] = self.get(k, 0) + int(v)
            elif isinstance(v, float):
                self[k] = max(self.get(k, 0.0), v)
        return self


def compare_slice(x: np.ndarray, q: np.ndarray, t0: int, B: int, C: float,
                  g_words: np.ndarray, g_hnorm: np.ndarray, g_pos: np.ndarray | None,
                  g_val: np.ndarray | None, g_y: np.ndarray | None, S: int,
                  out_f32: bool, npack: bool = False, exact: bool = False) -> Report:
    """Compare the GPU records of tokens [t0, t0+T) of one slice with the
    oracle.  x: [T, D] input values; g_*: the GPU's records for the same
    tokens (g_pos/g_val: the side-list entries of those batches; g_hnorm:
    [T, cpt] binary16 codes, or with npack the [T, W] packed norm words;
    with exact, g_words are the [ceil(T / 4), group words] groups (t0 a
    multiple of 4) and g_hnorm is unused)."""
    T, D = x.shape
    cpt = D // 4
    b = O.code_bits(S)
    W = O.words_per_row(S, D)
    rep = Report(chunks=T * cpt, exempt=0, code_mismatch=0, outliers=0)
    ref = O.encode_range(x, q, t0, B, C)
    codes_o = ref["codes"].reshape(T, cpt)
    hn_o = ref["hnorm"].reshape(T, cpt)
    gap = ref["gap"].reshape(T, cpt)

    exact_groups = None
    if exact:
        # norm codes (24 S levels) bit-exact; the decode below then uses the
        # half-norm records those codes stand for
        assert t0 % O.EXACT_ROWS == 0
        nc_o = O.exact_norms(hn_o, S)
        exact_groups = np.asarray(g_words).view(np.uint32).reshape(-1, O.exact_group_words(cpt, S))
        codes_g, nc_g = O.unpack_exact(exact_groups, T, cpt, S)
        bad = np.argwhere(nc_g != nc_o)
        assert bad.size == 0, \
            f"exact norm code differs at {bad[:5].tolist()}: gpu {nc_g[tuple(bad[0])]} oracle {nc_o[tuple(bad[0])]}"
        hn_o = O.exact_norm_to_h16(nc_o, S)
    elif npack:
        # compact norm codes (and their packed words): bit-exact; the decode
        # below then uses the half-norm records those codes stand for
        nc_o = O.compact_norms(hn_o, b)
        wg = np.asarray(g_hnorm).view(np.uint32).reshape(T, W)
        nc_g = unpack_words(wg, cpt, b)
        bad = np.argwhere(nc_g != nc_o)
        assert bad.size == 0, \
            f"norm code differs at {bad[:5].tolist()}: gpu {nc_g[tuple(bad[0])]:#x} oracle {nc_o[tuple(bad[0])]:#x}"
        np.testing.assert_array_equal(wg, np.stack([O.pack_row(nc_o[t], b, W) for t in range(T)]))
        hn_o = O.compact_to_h16(nc_o, b)
    else:
        # half-norm codes and flags: bit-exact
        hn_g = np.asarray(g_hnorm).reshape(T, cpt).view(np.uint16)
        bad = np.argwhere(hn_g != hn_o)
        assert bad.size == 0, \
            f"hnorm differs at {bad[:5].tolist()}: gpu {hn_g[tuple(bad[0])]:#x} oracle {hn_o[tuple(bad[0])]:#x}"

    # side list: bit-exact
    if B > 0:
        rep["outliers"] = len(ref["side_pos"])
        assert g_pos is not None and len(g_pos) == len(ref["side_pos"]), \
            f"outlier count gpu {None if g_pos is None else len(g_pos)} oracle {len(ref['side_pos'])}"
        np.testing.assert_array_equal(np.asarray(g_pos).view(np.uint32), ref["side_pos"])
        np.testing.assert_array_equal(np.asarray(g_val).view(np.uint16).reshape(-1, 4), ref["side_val"])

    # codes: exact outside near ties; near ties must be near-optimal
    if not exact:
        codes_g = unpack_words(np.asarray(g_words).view(np.uint32).reshape(T, W), cpt, b)
    assert codes_g.max(initial=0) < 24 * S
    diff = codes_g != codes_o
    exempt = gap < GAP_EXEMPT
    rep["exempt"] = int(exempt.sum())
    rep["code_mismatch"] = int(diff.sum())
    hard = diff & ~exempt
    if hard.any():
        t, c = np.argwhere(hard)[0]
        raise AssertionError(f"code differs outside the near-tie band at token {t0 + t} chunk {c}: "
                             f"gpu {codes_g[t, c]} oracle {codes_o[t, c]} gap {gap[t, c]:.3e}")
    cw = None
    if diff.any():
        cw = codeword_table(q)
        xs = x.reshape(T, cpt, 4).astype(np.float64)
        for t, c in np.argwhere(diff):
            u = xs[t, c] / np.linalg.norm(xs[t, c])
            best = cw[codes_o[t, c]] @ u
            mine = cw[codes_g[t, c]] @ u
            assert mine >= best - GAP_EXEMPT, f"near-tie code not near-optimal at {t0 + t},{c}"
    if exact:
        # group words bit-exact in groups whose index codes all match
        ng = exact_groups.shape[0]
        pad = ng * O.EXACT_ROWS - T
        dpad = np.concatenate([diff, np.zeros((pad, cpt), bool)]) if pad else diff
        groups_ok = ~dpad.reshape(ng, -1).any(axis=1)
        words_o = O.pack_exact(codes_o, O.exact_norms(ref["hnorm"].reshape(T, cpt), S), S)
        np.testing.assert_array_equal(exact_groups[groups_ok], words_o[groups_ok])
    else:
        # packed words bit-exact on rows whose codes match
        rows_ok = ~diff.any(axis=1)
        words_o = np.stack([O.pack_row(codes_o[t], b, W) for t in np.flatnonzero(rows_ok)]) if rows_ok.any() else None
        if words_o is not None:
            np.testing.assert_array_equal(np.asarray(g_words).view(np.uint32).reshape(T, W)[rows_ok], words_o)

    # decoded values
    if g_y is not None:
        y_o = O.decode_range(codes_o.reshape(-1), hn_o.reshape(-1), T, D, q,
                             ref["side_pos"] if B > 0 else None,
                             ref["side_val"] if B > 0 else None, t0)
        yg = np.asarray(g_y).astype(np.float64).reshape(T, cpt, 4)
        yo = y_o.reshape(T, cpt, 4)
        if diff.any():
            for t, c in np.argwhere(diff):
                r = 2.0 * float(np.float16(np.uint16(hn_o[t, c] & 0x7FFF).view(np.float16)))
                yo[t, c] = r * cw[codes_g[t, c]]
        # the oracle's output is its fp64 value rounded to the output type
        if out_f32:
            yo = O.round_f32(yo).astype(np.float64).reshape(T, cpt, 4)
        else:
            yo = O.round_f16(yo).view(np.float16).astype(np.float64).reshape(T, cpt, 4)
        rhat = 2.0 * (hn_o & 0x7FFF).view(np.float16).astype(np.float64)
        # (identical values, infinities of the binary16 overflow included, differ by 0)
        err = np.where(yg == yo, 0.0, np.abs(yg - yo)).max(axis=2)
        flagged = (hn_o & 0x8000) != 0
        # 1e-3 of the chunk norm; binary16 outputs below the normal range
        # cannot resolve finer than one subnormal step (2^-24)
        lim = REL_TOL * rhat if out_f32 else np.maximum(REL_TOL * rhat, 2.0 ** -24)
        worst = np.argmax(np.where(flagged, 0, err - lim))
        t, c = np.unravel_index(worst, err.shape)
        assert np.all(err[~flagged] <= lim[~flagged]), \
            f"decode error {err[t, c]:.3e} > {lim[t, c]:.3e} at {t0 + t},{c}"
        if flagged.any():
            np.testing.assert_array_equal(yg[flagged], x.reshape(T, cpt, 4)[flagged].astype(np.float16).astype(np.float64))
        nz = rhat > 0
        rep["max_rel_err"] = float((err[nz & ~flagged] / rhat[nz & ~flagged]).max(initial=0.0))
    return rep
