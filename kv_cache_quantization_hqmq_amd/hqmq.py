"""ctypes binding of the HQMQ C ABI (include/hqmq.h).

Argument marshalling only: every step of the codec runs in the HIP kernels of
libhqmq.so.  PyTorch supplies device memory (``tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``).  The functions keep the
C names; ``Desc``/``Records`` are the C structs, and ``allocate_records`` /
``workspace`` size torch buffers from ``hqmq_sizes``.

There is no fallback: if libhqmq.so is missing or no GPU is visible, calls
that need the device raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HQMQ_LIB selects another build of the same library (the host-sanitizer
# build, or a build kept for a comparison run)
LIB_PATH = os.environ.get("HQMQ_LIB") or os.path.join(_HERE, "libhqmq.so")

HQMQ_OK, HQMQ_EINVAL, HQMQ_ENOTSUP, HQMQ_ECAPACITY, HQMQ_EHIP = 0, -1, -2, -3, -4
HQMQ_F16, HQMQ_F32 = 0, 1
HQMQ_ROLE_K, HQMQ_ROLE_V = 0, 1
HQMQ_NORM_F16, HQMQ_NORM_PACKED, HQMQ_NORM_EXACT = 0, 1, 2

# every symbol include/hqmq.h declares
EXPORTS = ("hqmq_strerror", "hqmq_sizes", "hqmq_make_codebook", "hqmq_encode",
           "hqmq_encode_timed", "hqmq_encode_result", "hqmq_decode", "hqmq_attn_sizes",
           "hqmq_attend", "hqmq_attend_noalloc", "hqmq_paged_sizes", "hqmq_paged_clear", "hqmq_append",
           "hqmq_attend_paged", "hqmq_set_search_blocks_per_cu",
           "hqmq_ceiling_stream", "hqmq_ceiling_compute")

# include/hqmq_ceiling.h
HQMQ_CEIL_READ, HQMQ_CEIL_WRITE, HQMQ_CEIL_COPY = 0, 1, 2
HQMQ_CEIL_FMA_F32, HQMQ_CEIL_MFMA_F32, HQMQ_CEIL_MFMA_F16 = 0, 1, 2


class HQMQError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {hqmq_strerror(code)} ({code})")
        self.code = code


class CapacityError(HQMQError):
    def __init__(self, needed: int):
        super().__init__(HQMQ_ECAPACITY, "hqmq_encode_result")
        self.needed = needed


class Desc(ctypes.Structure):
    """hqmq_desc."""
    _fields_ = [("layers", ctypes.c_int64), ("kv_heads", ctypes.c_int64),
                ("tokens", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("S", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("med_batch_tokens", ctypes.c_int64), ("med_C", ctypes.c_float),
                ("norm_format", ctypes.c_int32)]

    @classmethod
    def make(cls, layers, kv_heads, tokens, head_dim, S, dtype=HQMQ_F16,
             med_batch_tokens=0, med_C=3.0, norm_format=HQMQ_NORM_F16) -> "Desc":
        return cls(layers, kv_heads, tokens, head_dim, S, dtype, med_batch_tokens, med_C, norm_format)

    @property
    def shape(self):
        return (self.layers, self.kv_heads, self.tokens, self.head_dim)


class Sizes(ctypes.Structure):
    """hqmq_sizes_t."""
    _fields_ = [("code_bits", ctypes.c_int32), ("words_per_token", ctypes.c_int32),
                ("chunks", ctypes.c_int64), ("batches", ctypes.c_int64),
                ("max_outliers", ctypes.c_int64), ("input_bytes", ctypes.c_uint64),
                ("idx_bytes", ctypes.c_uint64), ("hnorm_bytes", ctypes.c_uint64),
                ("offsets_bytes", ctypes.c_uint64), ("side_entry_bytes", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64), ("codebook_bytes", ctypes.c_uint64),
                ("group_rows", ctypes.c_int32), ("group_words", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class Enc(ctypes.Structure):
    """hqmq_enc (device pointers)."""
    _fields_ = [("idx", ctypes.c_void_p), ("hnorm", ctypes.c_void_p),
                ("batch_offsets", ctypes.c_void_p), ("out_pos", ctypes.c_void_p),
                ("out_val", ctypes.c_void_p), ("out_capacity", ctypes.c_uint64),
                ("status", ctypes.c_void_p)]


class AttnDesc(ctypes.Structure):
    """hqmq_attn_desc."""
    _fields_ = [("batch", ctypes.c_int32), ("group", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("scale", ctypes.c_float), ("reserved", ctypes.c_int32)]

    @classmethod
    def make(cls, batch, group, layer, max_len, scale) -> "AttnDesc":
        return cls(batch, group, layer, max_len, scale, 0)


class AttnSizes(ctypes.Structure):
    """hqmq_attn_sizes_t."""
    _fields_ = [("workspace_bytes", ctypes.c_uint64), ("splits", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32)]


class PagedDesc(ctypes.Structure):
    """hqmq_paged_desc."""
    _fields_ = [("num_pages", ctypes.c_int64), ("page_tokens", ctypes.c_int32),
                ("page_capacity", ctypes.c_int32)]


class Pages(ctypes.Structure):
    """hqmq_pages."""
    _fields_ = [("idx", ctypes.c_void_p), ("hnorm", ctypes.c_void_p), ("side_count", ctypes.c_void_p),
                ("side_pos", ctypes.c_void_p), ("side_val", ctypes.c_void_p)]


class PagedSizes(ctypes.Structure):
    """hqmq_paged_sizes_t."""
    _fields_ = [("idx_bytes", ctypes.c_uint64), ("hnorm_bytes", ctypes.c_uint64),
                ("side_count_bytes", ctypes.c_uint64), ("side_pos_bytes", ctypes.c_uint64),
                ("side_val_bytes", ctypes.c_uint64), ("append_workspace_bytes", ctypes.c_uint64)]


_lib = None


def lib():
    """The loaded libhqmq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_quantization_hqmq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.hqmq_strerror.argtypes = [ctypes.c_int]
        L.hqmq_strerror.restype = ctypes.c_char_p
        L.hqmq_sizes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Sizes)]
        L.hqmq_make_codebook.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_float)]
        L.hqmq_encode.argtypes = [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(Enc), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
        L.hqmq_encode_timed.argtypes = [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.POINTER(Enc), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.hqmq_encode_result.argtypes = [ctypes.POINTER(Enc), ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_uint64)]
        L.hqmq_decode.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Enc), ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
        L.hqmq_attn_sizes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(AttnDesc),
                                      ctypes.POINTER(AttnSizes)]
        L.hqmq_attend.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(AttnDesc), ctypes.POINTER(Enc),
                                  ctypes.c_void_p, ctypes.POINTER(Enc), ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.hqmq_attend_noalloc.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(AttnDesc), ctypes.POINTER(Enc),
                                          ctypes.c_void_p, ctypes.POINTER(Enc), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
        L.hqmq_paged_sizes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(PagedDesc),
                                       ctypes.POINTER(PagedSizes)]
        L.hqmq_paged_clear.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(PagedDesc), ctypes.POINTER(Pages),
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.hqmq_append.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(PagedDesc), ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Pages), ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.hqmq_attend_paged.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(PagedDesc),
                                        ctypes.POINTER(AttnDesc), ctypes.POINTER(Pages), ctypes.c_void_p,
                                        ctypes.POINTER(Pages), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.hqmq_set_search_blocks_per_cu.argtypes = [ctypes.c_int32]
        L.hqmq_ceiling_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]
        L.hqmq_ceiling_compute.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_double)]
        for f in ("hqmq_sizes", "hqmq_make_codebook", "hqmq_encode", "hqmq_encode_timed",
                  "hqmq_encode_result", "hqmq_decode", "hqmq_attn_sizes", "hqmq_attend", "hqmq_attend_noalloc",
                  "hqmq_paged_sizes", "hqmq_paged_clear", "hqmq_append", "hqmq_attend_paged",
                  "hqmq_set_search_blocks_per_cu", "hqmq_ceiling_stream", "hqmq_ceiling_compute"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != HQMQ_OK:
        raise HQMQError(rc, where)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


# ------------------------------------------------------------------ C calls
def hqmq_strerror(code: int) -> str:
    return lib().hqmq_strerror(int(code)).decode()


def hqmq_set_search_blocks_per_cu(n: int) -> None:
    """Cap the fp16 encode search's resident blocks per compute unit (0: no cap)."""
    _check(lib().hqmq_set_search_blocks_per_cu(int(n)), "hqmq_set_search_blocks_per_cu")


def hqmq_ceiling_stream(kind: int, src, dst, nbytes: int, stream=None) -> None:
    """One streaming pass (read, write or copy) of nbytes over device tensors."""
    _check(lib().hqmq_ceiling_stream(kind, _ptr(src), _ptr(dst), nbytes, _stream(stream)), "hqmq_ceiling_stream")


def hqmq_ceiling_compute(kind: int, iterations: int, sink, stream=None) -> float:
    """Launch an arithmetic ceiling loop; returns the flops it performs."""
    fl = ctypes.c_double(0.0)
    _check(lib().hqmq_ceiling_compute(kind, iterations, _ptr(sink), _stream(stream), ctypes.byref(fl)),
           "hqmq_ceiling_compute")
    return fl.value


def hqmq_sizes(desc: Desc) -> Sizes:
    out = Sizes()
    _check(lib().hqmq_sizes(ctypes.byref(desc), ctypes.byref(out)), "hqmq_sizes")
    return out


def hqmq_make_codebook(seed: int, layers: int, kv_heads: int, role: int, S: int) -> np.ndarray:
    """Host codebook [layers, kv_heads, S, 4] float32."""
    out = np.empty((layers, kv_heads, S, 4), np.float32)
    _check(lib().hqmq_make_codebook(seed, layers, kv_heads, role, S,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))),
           "hqmq_make_codebook")
    return out


def hqmq_encode(desc: Desc, x, codebook, rec: "Records", workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hqmq_encode(ctypes.byref(desc), _ptr(x), _ptr(codebook), ctypes.byref(rec.c),
                           _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "hqmq_encode")


def hqmq_encode_timed(desc: Desc, x, codebook, rec: "Records", workspace=None, stream=None,
                      search_begin=None, search_end=None) -> None:
    """hqmq_encode plus HIP events (raw hipEvent_t handles) recorded around
    the search kernel on the same stream."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hqmq_encode_timed(ctypes.byref(desc), _ptr(x), _ptr(codebook), ctypes.byref(rec.c),
                                 _ptr(workspace), ws_bytes, _stream(stream), search_begin,
                                 search_end)
    _check(rc, "hqmq_encode_timed")


def hqmq_encode_result(rec: "Records", stream=None) -> int:
    n = ctypes.c_uint64(0)
    rc = lib().hqmq_encode_result(ctypes.byref(rec.c), _stream(stream), ctypes.byref(n))
    if rc == HQMQ_ECAPACITY:
        raise CapacityError(int(n.value))
    _check(rc, "hqmq_encode_result")
    return int(n.value)


def hqmq_decode(desc: Desc, rec: "Records", codebook, y, stream=None) -> None:
    rc = lib().hqmq_decode(ctypes.byref(desc), ctypes.byref(rec.c), _ptr(codebook), _ptr(y),
                           _stream(stream))
    _check(rc, "hqmq_decode")


def hqmq_attn_sizes(desc: Desc, adesc: AttnDesc) -> AttnSizes:
    out = AttnSizes()
    _check(lib().hqmq_attn_sizes(ctypes.byref(desc), ctypes.byref(adesc), ctypes.byref(out)),
           "hqmq_attn_sizes")
    return out


def hqmq_attend(desc: Desc, adesc: AttnDesc, rec_k: "Records", codebook_k, rec_v: "Records",
                codebook_v, q, seq_start, seq_len, out, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hqmq_attend(ctypes.byref(desc), ctypes.byref(adesc), ctypes.byref(rec_k.c),
                           _ptr(codebook_k), ctypes.byref(rec_v.c), _ptr(codebook_v), _ptr(q),
                           _ptr(seq_start), _ptr(seq_len), _ptr(out), _ptr(workspace), ws_bytes,
                           _stream(stream))
    _check(rc, "hqmq_attend")


HQMQ_ATTEND_SCRATCH_BYTES = 16 << 20   # include/hqmq.h


def hqmq_attend_noalloc(desc: Desc, adesc: AttnDesc, rec_k: "Records", codebook_k, rec_v: "Records",
                        codebook_v, q, seq_start, seq_len, out, stream=None) -> None:
    """hqmq_attend with the library's own per-GPU scratch (no workspace)."""
    rc = lib().hqmq_attend_noalloc(ctypes.byref(desc), ctypes.byref(adesc), ctypes.byref(rec_k.c),
                                   _ptr(codebook_k), ctypes.byref(rec_v.c), _ptr(codebook_v), _ptr(q),
                                   _ptr(seq_start), _ptr(seq_len), _ptr(out), _stream(stream))
    _check(rc, "hqmq_attend_noalloc")


def hqmq_paged_sizes(desc: Desc, pdesc: PagedDesc) -> PagedSizes:
    out = PagedSizes()
    _check(lib().hqmq_paged_sizes(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(out)),
           "hqmq_paged_sizes")
    return out


def hqmq_paged_clear(desc: Desc, pdesc: PagedDesc, pool: "Pool", pages, stream=None) -> None:
    rc = lib().hqmq_paged_clear(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(pool.c), _ptr(pages),
                                int(pages.numel()), _stream(stream))
    _check(rc, "hqmq_paged_clear")


def hqmq_append(desc: Desc, pdesc: PagedDesc, x, slots, codebook, pool: "Pool", status=None,
                workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hqmq_append(ctypes.byref(desc), ctypes.byref(pdesc), _ptr(x), _ptr(slots), _ptr(codebook),
                           ctypes.byref(pool.c), _ptr(status), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "hqmq_append")


def hqmq_attend_paged(desc: Desc, pdesc: PagedDesc, adesc: AttnDesc, pool_k: "Pool", codebook_k,
                      pool_v: "Pool", codebook_v, q, page_table, seq_len, out, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hqmq_attend_paged(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(adesc),
                                 ctypes.byref(pool_k.c), _ptr(codebook_k), ctypes.byref(pool_v.c),
                                 _ptr(codebook_v), _ptr(q), _ptr(page_table), int(page_table.shape[1]),
                                 _ptr(seq_len), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "hqmq_attend_paged")


# ------------------------------------------------------------------ buffers
@dataclass
class Records:
    """Torch buffers of one encoded tensor plus the C struct pointing at them."""
    idx: object
    hnorm: object
    batch_offsets: object
    out_pos: object
    out_val: object
    status: object
    capacity: int
    c: Enc


def allocate_records(desc: Desc, capacity: int | None = None, device="cuda") -> Records:
    """Device buffers for ``desc``; ``capacity`` side-list entries (default:
    the worst case floor(n/2) per batch, capped at 1/8 of the chunks)."""
    import torch
    sz = hqmq_sizes(desc)
    T, W, cpt = desc.tokens, sz.words_per_token, desc.head_dim // 4
    L, H = desc.layers, desc.kv_heads
    if desc.norm_format == HQMQ_NORM_EXACT:   # groups of 4 token rows, no norm plane
        idx = torch.empty((L, H, (T + 3) // 4, sz.group_words), dtype=torch.int32, device=device)
        hnorm = None
    else:
        idx = torch.empty((L, H, T, W), dtype=torch.int32, device=device)
    if desc.norm_format == HQMQ_NORM_PACKED:   # u32 words laid out like idx
        hnorm = torch.empty((L, H, T, W), dtype=torch.int32, device=device)
    elif desc.norm_format == HQMQ_NORM_F16:
        hnorm = torch.empty((L, H, T, cpt), dtype=torch.int16, device=device)
    med = desc.med_batch_tokens > 0
    if capacity is None:
        capacity = min(sz.max_outliers, max(1, sz.chunks // 8)) if med else 0
    capacity = int(capacity) if med else 0
    offs = torch.empty((sz.batches + 1,), dtype=torch.int64, device=device) if med else None
    pos = torch.empty((max(capacity, 1),), dtype=torch.int32, device=device) if med else None
    val = torch.empty((max(capacity, 1), 4), dtype=torch.int16, device=device) if med else None
    status = torch.zeros((2,), dtype=torch.int64, device=device)
    c = Enc(_ptr(idx), _ptr(hnorm), _ptr(offs), _ptr(pos), _ptr(val), capacity, _ptr(status))
    return Records(idx, hnorm, offs, pos, val, status, capacity, c)


def workspace(desc: Desc, device="cuda"):
    import torch
    n = hqmq_sizes(desc).workspace_bytes
    return torch.empty((max(int(n), 1),), dtype=torch.uint8, device=device) if n else None


def encode(desc: Desc, x, codebook, capacity: int | None = None, ws=None, stream=None) -> Records:
    """Encode ``x`` and wait for the outlier count; on side-list overflow,
    re-allocate with the reported size and encode again."""
    if ws is None:
        ws = workspace(desc, x.device)
    rec = allocate_records(desc, capacity, x.device)
    hqmq_encode(desc, x, codebook, rec, ws, stream)
    try:
        rec.n_outliers = hqmq_encode_result(rec, stream)
    except CapacityError as e:
        rec = allocate_records(desc, e.needed, x.device)
        hqmq_encode(desc, x, codebook, rec, ws, stream)
        rec.n_outliers = hqmq_encode_result(rec, stream)
    return rec


def decode(desc: Desc, rec: Records, codebook, y=None, stream=None):
    import torch
    if y is None:
        dt = torch.float32 if desc.dtype == HQMQ_F32 else torch.float16
        y = torch.empty(desc.shape, dtype=dt, device=rec.idx.device)
    hqmq_decode(desc, rec, codebook, y, stream)
    return y


def attend(desc: Desc, layer: int, rec_k: Records, codebook_k, rec_v: Records, codebook_v, q,
           seq_start, seq_len, max_len: int, scale: float | None = None, out=None, ws=None,
           stream=None):
    """Decode-step attention over one layer of an encoded cache.  q is
    [batch, kv_heads * group, head_dim] fp16 on the device; seq_start (int64)
    and seq_len (int32) are device tensors of length batch.  Returns out
    [batch, kv_heads * group, head_dim] fp32."""
    import math
    import torch
    batch, hq, D = q.shape
    group = hq // desc.kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    a = AttnDesc.make(batch, group, layer, max_len, scale)
    if ws is None:
        n = hqmq_attn_sizes(desc, a).workspace_bytes
        ws = torch.empty((max(int(n), 16),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, hq, D), dtype=torch.float32, device=q.device)
    hqmq_attend(desc, a, rec_k, codebook_k, rec_v, codebook_v, q, seq_start, seq_len, out, ws, stream)
    return out


# ------------------------------------------------------------------ paged pool
@dataclass
class Pool:
    """Torch buffers of one role's paged pool plus the C struct pointing at them."""
    idx: object
    hnorm: object
    side_count: object
    side_pos: object
    side_val: object
    c: Pages


def allocate_pool(desc: Desc, pdesc: PagedDesc, device="cuda") -> Pool:
    """A pool for ``desc``'s codec and ``pdesc``'s pages, every page empty."""
    import torch
    sz = hqmq_sizes(desc)
    L, H, D = desc.layers, desc.kv_heads, desc.head_dim
    NP, P, cap = pdesc.num_pages, pdesc.page_tokens, pdesc.page_capacity
    W = sz.words_per_token
    idx = torch.empty((L, H, NP, P, W), dtype=torch.int32, device=device)
    if desc.norm_format == HQMQ_NORM_PACKED:
        hnorm = torch.empty((L, H, NP, P, W), dtype=torch.int32, device=device)
    else:
        hnorm = torch.empty((L, H, NP, P, D // 4), dtype=torch.int16, device=device)
    count = torch.zeros((L, H, NP), dtype=torch.int32, device=device)
    pos = torch.empty((L, H, NP, max(cap, 1)), dtype=torch.int32, device=device)
    val = torch.empty((L, H, NP, max(cap, 1), 4), dtype=torch.int16, device=device)
    c = Pages(_ptr(idx), _ptr(hnorm), _ptr(count), _ptr(pos), _ptr(val))
    return Pool(idx, hnorm, count, pos, val, c)


def append_workspace(desc: Desc, pdesc: PagedDesc, device="cuda"):
    """Workspace of an append of ``desc.tokens`` tokens."""
    import torch
    n = hqmq_paged_sizes(desc, pdesc).append_workspace_bytes
    return torch.empty((max(int(n), 1),), dtype=torch.uint8, device=device)


def append(desc: Desc, pdesc: PagedDesc, pool: Pool, x, slots, codebook, ws=None, status=None,
           stream=None) -> None:
    """Append x [layers, kv_heads, T, head_dim] to ``pool`` at ``slots`` (int64
    device tensor of T slots); ``desc.tokens`` must be T."""
    if ws is None:
        ws = append_workspace(desc, pdesc, x.device)
    hqmq_append(desc, pdesc, x, slots, codebook, pool, status, ws, stream)


def attend_paged(desc: Desc, pdesc: PagedDesc, layer: int, pool_k: Pool, codebook_k, pool_v: Pool, codebook_v,
                 q, page_table, seq_len, max_len: int, scale: float | None = None, out=None, ws=None,
                 stream=None):
    """Decode-step attention over paged pools: page_table [batch, max_pages]
    int32 and seq_len [batch] int32 device tensors; returns out [batch,
    kv_heads * group, head_dim] fp32."""
    import math
    import torch
    batch, hq, D = q.shape
    group = hq // desc.kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    a = AttnDesc.make(batch, group, layer, max_len, scale)
    if ws is None:
        n = hqmq_attn_sizes(desc, a).workspace_bytes
        ws = torch.empty((max(int(n), 16),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, hq, D), dtype=torch.float32, device=q.device)
    hqmq_attend_paged(desc, pdesc, a, pool_k, codebook_k, pool_v, codebook_v, q, page_table, seq_len, out, ws,
                      stream)
    return out
