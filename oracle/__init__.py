"""HQMQ oracle: ctypes front end of the plain-C reference in hqmq_oracle.c.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It never
imports the HIP library or its Python binding, and the HIP library never
imports it.

Every function below is marshalling around the C function of the same name
(prefixed ``or_`` there); the arithmetic and its citations live in the C
file.  The tensor-level helpers (``encode_tensor``/``decode_tensor``) only
loop over (layer, head) slices and lay the per-slice results out the way the
library's records are laid out, so that tests can compare them directly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HQMQ_ORACLE_LIB: another build of the same source (the host sanitizer run)
_LIB_PATH = os.environ.get("HQMQ_ORACLE_LIB") or os.path.join(_HERE, "libhqmq_oracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u64p = ctypes.POINTER(ctypes.c_uint64)


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager: route every wrapper in this module to another build
    of the oracle (the tests use it to check that planted mistakes in a
    copy of the C source are caught by the pins)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _configure(L):
    L.or_qmul.argtypes = [_f64p, _f64p, _f64p]
    L.or_t2_element.argtypes = [ctypes.c_int, _f64p]
    L.or_f16_bits.argtypes = [ctypes.c_double]
    L.or_f16_bits.restype = ctypes.c_uint16
    L.or_f16_value.argtypes = [ctypes.c_uint16]
    L.or_f16_value.restype = ctypes.c_double
    L.or_philox4x64_10.argtypes = [_u64p, _u64p, _u64p]
    L.or_make_codebook.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, _f32p]
    L.or_codebook_value.argtypes = [ctypes.c_float]
    L.or_codebook_value.restype = ctypes.c_double
    L.or_norm2.argtypes = [_f32p]
    L.or_norm2.restype = ctypes.c_float
    L.or_half_norm_bits.argtypes = [ctypes.c_float]
    L.or_half_norm_bits.restype = ctypes.c_uint16
    L.or_codeword.argtypes = [_f32p, ctypes.c_int, _f64p]
    L.or_nearest.argtypes = [_f32p, _f32p, ctypes.c_int, _i32p, _f64p]
    L.or_lower_median.argtypes = [_f32p, ctypes.c_int64]
    L.or_lower_median.restype = ctypes.c_float
    L.or_med3_threshold.argtypes = [ctypes.c_float, ctypes.c_float]
    L.or_med3_threshold.restype = ctypes.c_float
    L.or_code_bits.argtypes = [ctypes.c_int]
    L.or_code_bits.restype = ctypes.c_int
    L.or_pack_row.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _u32p, ctypes.c_int]
    L.or_unpack_row.argtypes = [_u32p, ctypes.c_int, ctypes.c_int, _i32p]
    L.or_encode_range.argtypes = [
        _f32p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
        _f32p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
        _i32p, _u16p, _f64p, _f32p,
        _u32p, _u16p, ctypes.c_int64, _i64p]
    L.or_encode_range.restype = ctypes.c_int64
    L.or_decode_range.argtypes = [
        _i32p, _u16p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
        _f32p, ctypes.c_int, _u32p, _u16p, ctypes.c_int64, _f64p]
    L.or_decode_range.restype = ctypes.c_int64
    L.or_round_f32.argtypes = [_f64p, ctypes.c_int64, _f32p]
    L.or_round_f16.argtypes = [_f64p, ctypes.c_int64, _u16p]
    L.or_num_threads.restype = ctypes.c_int
    L.or_compact_norm.argtypes = [ctypes.c_uint16, ctypes.c_int]
    L.or_compact_norm.restype = ctypes.c_uint32
    L.or_compact_to_h16.argtypes = [ctypes.c_uint32, ctypes.c_int]
    L.or_compact_to_h16.restype = ctypes.c_uint16
    L.or_compact_norms.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int, _u32p]
    L.or_exact_m.argtypes = [ctypes.c_int]
    L.or_exact_m.restype = ctypes.c_int
    L.or_exact_level_pattern.argtypes = [ctypes.c_uint32, ctypes.c_int]
    L.or_exact_level_pattern.restype = ctypes.c_uint32
    L.or_exact_norm.argtypes = [ctypes.c_uint16, ctypes.c_int]
    L.or_exact_norm.restype = ctypes.c_uint32
    L.or_exact_norm_to_h16.argtypes = [ctypes.c_uint32, ctypes.c_int]
    L.or_exact_norm_to_h16.restype = ctypes.c_uint16
    L.or_exact_norms.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int, _u32p]
    L.or_exact_group_words.argtypes = [ctypes.c_int, ctypes.c_int]
    L.or_exact_group_words.restype = ctypes.c_int
    L.or_pack_exact_group.argtypes = [_i32p, _u32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u32p]
    L.or_unpack_exact_group.argtypes = [_u32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _u32p]
    L.or_attend.argtypes = [_f64p, _f64p, ctypes.c_int64, ctypes.c_int, _f64p, ctypes.c_int,
                            ctypes.c_double, _f64p]
    return L


# --------------------------------------------------------------- algebra
def qmul(a, b) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    out = np.empty(4, np.float64)
    lib().or_qmul(_p(a, _f64p), _p(b, _f64p), _p(out, _f64p))
    return out


def t2_element(p: int) -> np.ndarray:
    out = np.empty(4, np.float64)
    lib().or_t2_element(int(p), _p(out, _f64p))
    return out


def t2_elements() -> np.ndarray:
    return np.stack([t2_element(p) for p in range(24)])


# --------------------------------------------------------------- binary16
def f16_bits(v: float) -> int:
    return int(lib().or_f16_bits(float(v)))


def f16_value(h: int) -> float:
    return float(lib().or_f16_value(int(h)))


def round_f16(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.uint16)
    lib().or_round_f16(_p(y, _f64p), y.size, _p(out, _u16p))
    return out


def round_f32(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.float32)
    lib().or_round_f32(_p(y, _f64p), y.size, _p(out, _f32p))
    return out


# --------------------------------------------------------------- codebook
def philox4x64_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.empty(4, np.uint64)
    lib().or_philox4x64_10(_p(c, _u64p), _p(k, _u64p), _p(out, _u64p))
    return out


def codebook_value(q: float) -> float:
    return float(lib().or_codebook_value(float(np.float32(q))))


def make_codebook(seed: int, layers: int, heads: int, role: int, S: int) -> np.ndarray:
    out = np.empty((layers, heads, S, 4), np.float32)
    lib().or_make_codebook(int(seed), layers, heads, role, S, _p(out, _f32p))
    return out


# --------------------------------------------------------------- per chunk
def norm2(v) -> np.float32:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return np.float32(lib().or_norm2(_p(v, _f32p)))


def half_norm_bits(s2: float) -> int:
    return int(lib().or_half_norm_bits(float(np.float32(s2))))


def codeword(q, k: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(4, np.float64)
    lib().or_codeword(_p(q, _f32p), int(k), _p(out, _f64p))
    return out


def nearest(x, q):
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.zeros(1, np.int32)
    g = np.zeros(1, np.float64)
    lib().or_nearest(_p(x, _f32p), _p(q, _f32p), q.shape[0], _p(k, _i32p), _p(g, _f64p))
    return int(k[0]), float(g[0])


def lower_median(keys) -> np.float32:
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    return np.float32(lib().or_lower_median(_p(keys, _f32p), keys.size))


def med3_threshold(med: float, C: float = 3.0) -> np.float32:
    return np.float32(lib().or_med3_threshold(float(np.float32(med)), float(np.float32(C))))


def code_bits(S: int) -> int:
    return int(lib().or_code_bits(int(S)))


def words_per_row(S: int, D: int) -> int:
    return (code_bits(S) * (D // 4) + 31) // 32


def pack_row(codes, b: int, W: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    out = np.empty(W, np.uint32)
    lib().or_pack_row(_p(codes, _i32p), codes.size, b, _p(out, _u32p), W)
    return out


def unpack_row(words, cpt: int, b: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.empty(cpt, np.int32)
    lib().or_unpack_row(_p(words, _u32p), cpt, b, _p(out, _i32p))
    return out


# --------------------------------------------------------------- slices
def encode_range(x, q, t0: int = 0, B: int = 0, C: float = 3.0) -> dict:
    """Encode tokens [t0, t0+T) of one slice.  x: [T, D] (fp16 or fp32)."""
    x = np.ascontiguousarray(np.asarray(x).astype(np.float32))
    q = np.ascontiguousarray(q, dtype=np.float32)
    T, D = x.shape
    S = q.shape[0]
    n = T * (D // 4)
    codes = np.empty(n, np.int32)
    hnorm = np.empty(n, np.uint16)
    gap = np.empty(n, np.float64)
    s2 = np.empty(n, np.float32)
    # at most floor(n / 2) outliers per batch when fl(C C) >= 1, every chunk otherwise
    cap = n // 2 + 1 if np.float32(C) * np.float32(C) >= np.float32(1.0) else n
    side_pos = np.empty(cap, np.uint32)
    side_val = np.empty((cap, 4), np.uint16)
    nb = (T + B - 1) // B if B > 0 else 0
    counts = np.zeros(max(nb, 1), np.int64)
    r = lib().or_encode_range(
        _p(x, _f32p), T, D, t0, _p(q, _f32p), S, B, float(C),
        _p(codes, _i32p), _p(hnorm, _u16p), _p(gap, _f64p), _p(s2, _f32p),
        _p(side_pos, _u32p), _p(side_val, _u16p), cap, _p(counts, _i64p))
    if r < 0:
        raise ValueError("or_encode_range rejected its arguments")
    return dict(codes=codes, hnorm=hnorm, gap=gap, s2=s2,
                side_pos=side_pos[:r].copy(), side_val=side_val[:r].copy(),
                batch_counts=counts[:nb].copy())


def decode_range(codes, hnorm, T: int, D: int, q, side_pos=None, side_val=None,
                 t0: int = 0) -> np.ndarray:
    """Decode one slice's token range to fp64 values [T, D]."""
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    hnorm = np.ascontiguousarray(hnorm, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.float32)
    if side_pos is None:
        side_pos = np.zeros(1, np.uint32)
        side_val = np.zeros((1, 4), np.uint16)
        n_side = 0
    else:
        n_side = len(side_pos)
        side_pos = np.ascontiguousarray(side_pos, dtype=np.uint32)
        side_val = np.ascontiguousarray(side_val, dtype=np.uint16)
        if n_side == 0:
            side_pos = np.zeros(1, np.uint32)
            side_val = np.zeros((1, 4), np.uint16)
    y = np.empty((T, D), np.float64)
    r = lib().or_decode_range(_p(codes, _i32p), _p(hnorm, _u16p), T, D, t0,
                              _p(q, _f32p), q.shape[0], _p(side_pos, _u32p),
                              _p(side_val, _u16p), n_side, _p(y, _f64p))
    if r < 0:
        raise ValueError("or_decode_range: inconsistent records")
    return y


def compact_norms(h16, b: int) -> np.ndarray:
    """Compact norm codes (b bits) of binary16 half-norm records."""
    h = np.ascontiguousarray(h16, dtype=np.uint16)
    out = np.empty(h.shape, np.uint32)
    lib().or_compact_norms(_p(h, _u16p), h.size, int(b), _p(out, _u32p))
    return out


def compact_to_h16(codes, b: int) -> np.ndarray:
    """Half-norm records (binary16 pattern, or the flag) of compact codes."""
    c = np.asarray(codes, dtype=np.uint32).ravel()
    return np.array([lib().or_compact_to_h16(int(v), int(b)) for v in c], np.uint16).reshape(np.shape(codes))


EXACT_ROWS = 4   # token rows per exact-rate group


def exact_m(S: int) -> int:
    """m with 24 S = 3 2^m (-1 when S is not a power of two up to 1024)."""
    return int(lib().or_exact_m(int(S)))


def exact_level_pattern(n: int, S: int) -> int:
    return int(lib().or_exact_level_pattern(int(n), int(S)))


def exact_norm(h16: int, S: int) -> int:
    return int(lib().or_exact_norm(int(h16), int(S)))


def exact_norms(h16, S: int) -> np.ndarray:
    """Exact-rate norm codes (24 S levels) of binary16 half-norm records."""
    h = np.ascontiguousarray(h16, dtype=np.uint16)
    out = np.empty(h.shape, np.uint32)
    lib().or_exact_norms(_p(h, _u16p), h.size, int(S), _p(out, _u32p))
    return out


def exact_norm_to_h16(codes, S: int) -> np.ndarray:
    """Half-norm records (binary16 pattern, or the flag) of exact-rate norm codes."""
    c = np.asarray(codes, dtype=np.uint32).ravel()
    return np.array([lib().or_exact_norm_to_h16(int(v), int(S)) for v in c],
                    np.uint16).reshape(np.shape(codes))


def exact_group_words(cpt: int, S: int) -> int:
    return int(lib().or_exact_group_words(int(cpt), int(S)))


def pack_exact(codes, ncodes, S: int) -> np.ndarray:
    """Exact-rate records of T token rows: codes, ncodes [T, cpt] ->
    [ceil(T / 4), group words] u32 (one group per 4 rows, the last one
    zero-filled past row T)."""
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    ncodes = np.ascontiguousarray(ncodes, dtype=np.uint32)
    T, cpt = codes.shape
    gw = exact_group_words(cpt, S)
    ng = (T + EXACT_ROWS - 1) // EXACT_ROWS
    out = np.zeros((ng, gw), np.uint32)
    for g in range(ng):
        rows = min(EXACT_ROWS, T - EXACT_ROWS * g)
        c = np.ascontiguousarray(codes[EXACT_ROWS * g:EXACT_ROWS * g + rows])
        n = np.ascontiguousarray(ncodes[EXACT_ROWS * g:EXACT_ROWS * g + rows])
        w = np.zeros(gw, np.uint32)
        lib().or_pack_exact_group(_p(c, _i32p), _p(n, _u32p), rows, cpt, int(S), _p(w, _u32p))
        out[g] = w
    return out


def unpack_exact(words, T: int, cpt: int, S: int):
    """Inverse of pack_exact: (codes, ncodes), each [T, cpt]."""
    words = np.ascontiguousarray(words, dtype=np.uint32)
    codes = np.zeros((T, cpt), np.int32)
    ncodes = np.zeros((T, cpt), np.uint32)
    for g in range((T + EXACT_ROWS - 1) // EXACT_ROWS):
        rows = min(EXACT_ROWS, T - EXACT_ROWS * g)
        w = np.ascontiguousarray(words[g])
        c = np.zeros((rows, cpt), np.int32)
        n = np.zeros((rows, cpt), np.uint32)
        lib().or_unpack_exact_group(_p(w, _u32p), rows, cpt, int(S), _p(c, _i32p), _p(n, _u32p))
        codes[EXACT_ROWS * g:EXACT_ROWS * g + rows] = c
        ncodes[EXACT_ROWS * g:EXACT_ROWS * g + rows] = n
    return codes, ncodes


def attend(k, v, q, scale: float) -> np.ndarray:
    """Attention of query rows q [G, D] over k, v [T, D] (fp64): out [G, D]."""
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    q = np.ascontiguousarray(np.atleast_2d(q), dtype=np.float64)
    T, D = k.shape
    G = q.shape[0]
    out = np.empty((G, D), np.float64)
    if T == 0:
        out[:] = 0.0
        return out
    lib().or_attend(_p(k, _f64p), _p(v, _f64p), T, D, _p(q, _f64p), G, float(scale), _p(out, _f64p))
    return out


# --------------------------------------------------------------- tensors
def encode_tensor(x, codebook, B: int = 0, C: float = 3.0) -> dict:
    """Encode a whole [L, H, T, D] tensor slice by slice.

    Returns the records in the library's layout: ``idx`` [L, H, T, W] u32
    packed codes, ``hnorm`` [L, H, T, D/4] u16, ``codes`` (unpacked, same
    shape as hnorm), ``gap``, ``s2``, the side list concatenated in (slice,
    batch) order, ``batch_offsets`` (exclusive prefix, one per batch + 1).
    """
    x = np.asarray(x)
    L, H, T, D = x.shape
    S = codebook.shape[2]
    cpt = D // 4
    b = code_bits(S)
    W = words_per_row(S, D)
    idx = np.zeros((L, H, T, W), np.uint32)
    codes = np.zeros((L, H, T, cpt), np.int32)
    hnorm = np.zeros((L, H, T, cpt), np.uint16)
    gap = np.zeros((L, H, T, cpt), np.float64)
    s2 = np.zeros((L, H, T, cpt), np.float32)
    pos_l, val_l, cnt_l = [], [], []
    for l in range(L):
        for h in range(H):
            r = encode_range(x[l, h], codebook[l, h], 0, B, C)
            codes[l, h] = r["codes"].reshape(T, cpt)
            hnorm[l, h] = r["hnorm"].reshape(T, cpt)
            gap[l, h] = r["gap"].reshape(T, cpt)
            s2[l, h] = r["s2"].reshape(T, cpt)
            for t in range(T):
                idx[l, h, t] = pack_row(codes[l, h, t], b, W)
            pos_l.append(r["side_pos"])
            val_l.append(r["side_val"])
            cnt_l.append(r["batch_counts"])
    counts = np.concatenate(cnt_l) if cnt_l else np.zeros(0, np.int64)
    offsets = np.zeros(len(counts) + 1, np.uint64)
    offsets[1:] = np.cumsum(counts)
    return dict(idx=idx, codes=codes, hnorm=hnorm, gap=gap, s2=s2,
                side_pos=np.concatenate(pos_l), side_val=np.concatenate(val_l),
                batch_offsets=offsets, bits=b, words=W)


def decode_tensor(enc: dict, codebook, shape, B: int = 0) -> np.ndarray:
    """Decode oracle records of a whole tensor to fp64 [L, H, T, D]."""
    L, H, T, D = shape
    cpt = D // 4
    y = np.zeros((L, H, T, D), np.float64)
    nb = (T + B - 1) // B if B > 0 else 0
    off = enc["batch_offsets"].astype(np.int64)
    for l in range(L):
        for h in range(H):
            sl = l * H + h
            if nb > 0:
                e0, e1 = off[sl * nb], off[(sl + 1) * nb]
                sp, sv = enc["side_pos"][e0:e1], enc["side_val"][e0:e1]
            else:
                sp = sv = None
            y[l, h] = decode_range(enc["codes"][l, h].reshape(-1),
                                   enc["hnorm"][l, h].reshape(-1), T, D,
                                   codebook[l, h], sp, sv)
    return y


def num_threads() -> int:
    return int(lib().or_num_threads())
