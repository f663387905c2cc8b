"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every symbol include/hqmq.h declares, descriptors are validated
before anything is enqueued, buffer sizes follow the record layout, and the
codebook generator is bit-identical to the oracle's independent one."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import kv_cache_quantization_hqmq_amd as K
from kv_cache_quantization_hqmq_amd import hqmq as B
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hqmq.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(hqmq_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert declared == sorted(B.EXPORTS)
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_search_blocks_per_cu_accepts_0_to_7_only():
    """The scheduling setter takes 0 (no cap) to 7 and rejects anything else
    with HQMQ_EINVAL, leaving the setting as it was (host only, no GPU)."""
    lib = B.lib()
    try:
        for n in range(8):
            assert lib.hqmq_set_search_blocks_per_cu(n) == B.HQMQ_OK
        for n in (-1, 8, 64, -(2 ** 31)):
            assert lib.hqmq_set_search_blocks_per_cu(n) == B.HQMQ_EINVAL
        with pytest.raises(K.HQMQError):
            K.hqmq_set_search_blocks_per_cu(9)
    finally:
        K.hqmq_set_search_blocks_per_cu(0)


def test_struct_layouts_match_header(tmp_path):
    """Field offsets and sizes of the ctypes structs equal what a C compiler
    makes of include/hqmq.h."""
    structs = {"hqmq_desc": B.Desc, "hqmq_sizes_t": B.Sizes, "hqmq_enc": B.Enc,
               "hqmq_attn_desc": B.AttnDesc, "hqmq_attn_sizes_t": B.AttnSizes,
               "hqmq_paged_desc": B.PagedDesc, "hqmq_pages": B.Pages, "hqmq_paged_sizes_t": B.PagedSizes}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "hqmq.h"', "int main(void){"]
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def test_strerror():
    for c in (0, -1, -2, -3, -4, 7):
        assert isinstance(K.hqmq_strerror(c), str) and K.hqmq_strerror(c)


@pytest.mark.parametrize("field,value", [
    ("head_dim", 96), ("head_dim", 0), ("head_dim", 512), ("S", 0), ("S", 1025),
    ("dtype", 2), ("layers", -1), ("tokens", -5), ("med_batch_tokens", -1), ("norm_format", 3),
    ("norm_format", -1)])
def test_descriptor_validation(field, value):
    d = K.Desc.make(2, 2, 64, 128, 8, K.HQMQ_F16, 16, 3.0)
    setattr(d, field, value)
    with pytest.raises(K.HQMQError) as e:
        K.hqmq_sizes(d)
    assert e.value.code == B.HQMQ_EINVAL


def test_med_C_must_be_positive_when_med3_is_on():
    d = K.Desc.make(1, 1, 64, 128, 8, K.HQMQ_F16, 16, 0.0)
    with pytest.raises(K.HQMQError):
        K.hqmq_sizes(d)
    d.med_batch_tokens = 0
    K.hqmq_sizes(d)   # ignored when Med3x is off


def test_token_limit_for_u32_positions():
    d = K.Desc.make(1, 1, 2 ** 27, 128, 8, K.HQMQ_F16, 0, 3.0)
    with pytest.raises(K.HQMQError) as e:
        K.hqmq_sizes(d)
    assert e.value.code == B.HQMQ_ENOTSUP
    d.tokens = 2 ** 27 - 1
    K.hqmq_sizes(d)


def test_encode_rejects_before_enqueueing():
    """Validation errors come back synchronously; no device pointer is
    touched (null pointers here), so this runs without a GPU."""
    lib = B.lib()
    d = K.Desc.make(1, 1, 64, 128, 8, K.HQMQ_F16, 0, 3.0)
    enc = B.Enc()
    assert lib.hqmq_encode(ctypes.byref(d), None, None, ctypes.byref(enc), None, 0, None) == B.HQMQ_EINVAL
    assert lib.hqmq_decode(ctypes.byref(d), ctypes.byref(enc), None, None, None) == B.HQMQ_EINVAL
    assert lib.hqmq_encode(None, None, None, ctypes.byref(enc), None, 0, None) == B.HQMQ_EINVAL
    n = ctypes.c_uint64(5)
    assert lib.hqmq_encode_result(None, None, ctypes.byref(n)) == B.HQMQ_EINVAL
    # misaligned (but non-null) pointers
    d.med_batch_tokens = 16
    enc2 = B.Enc(16, 16, 16, 16, 16, 4, 16)
    assert lib.hqmq_encode(ctypes.byref(d), ctypes.c_void_p(18), ctypes.c_void_p(16),
                           ctypes.byref(enc2), ctypes.c_void_p(256), 1 << 20, None) == B.HQMQ_EINVAL
    # workspace too small
    assert lib.hqmq_encode(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(16),
                           ctypes.byref(enc2), ctypes.c_void_p(256), 16, None) == B.HQMQ_EINVAL


@pytest.mark.parametrize("L,H,T,D,S,dt,Bt", [
    (80, 8, 131072, 128, 32, 0, 4096), (32, 8, 32768, 128, 8, 0, 0), (1, 1, 4096, 128, 8, 1, 0),
    (2, 3, 1001, 64, 13, 0, 256), (1, 1, 0, 128, 8, 0, 64)])
def test_sizes_follow_the_layout(L, H, T, D, S, dt, Bt):
    d = K.Desc.make(L, H, T, D, S, dt, Bt, 3.0)
    s = K.hqmq_sizes(d)
    cpt = D // 4
    b = O.code_bits(S)
    W = (b * cpt + 31) // 32
    assert s.code_bits == b and s.words_per_token == W
    assert s.chunks == L * H * T * cpt
    assert s.idx_bytes == L * H * T * W * 4
    assert s.hnorm_bytes == s.chunks * 2
    assert s.input_bytes == s.chunks * 4 * (4 if dt == 1 else 2)
    assert s.codebook_bytes == L * H * S * 16
    if Bt > 0 and T > 0:
        Bc = min(Bt, T)
        nb = -(-T // Bc)
        assert s.batches == L * H * nb
        assert s.offsets_bytes == (s.batches + 1) * 8
        per = [min(Bc, T - i * Bc) * cpt // 2 for i in range(nb)]
        assert s.max_outliers == L * H * sum(per)
        assert s.workspace_bytes >= s.batches * (2048 * 4 + 4) + s.chunks // 8
    else:
        assert s.workspace_bytes == 0


@pytest.mark.parametrize("L,H,T,D,S,Bt", [
    (80, 8, 131072, 128, 32, 4096), (32, 8, 32768, 128, 8, 0), (2, 3, 1001, 64, 13, 256), (1, 1, 5, 16, 1, 0),
    (1, 2, 7, 256, 1024, 3)])
def test_sizes_packed_norms(L, H, T, D, S, Bt):
    """Packed norms: the norm plane has the index plane's size (b bits per
    chunk in the same row words), and the encode workspace adds a binary16
    half-norm plane (2 bytes per chunk) to what Med3x needs."""
    f16 = K.hqmq_sizes(K.Desc.make(L, H, T, D, S, K.HQMQ_F16, Bt, 3.0))
    pk = K.hqmq_sizes(K.Desc.make(L, H, T, D, S, K.HQMQ_F16, Bt, 3.0, K.HQMQ_NORM_PACKED))
    assert pk.hnorm_bytes == pk.idx_bytes == f16.idx_bytes
    assert pk.code_bits == f16.code_bits and pk.chunks == f16.chunks
    assert pk.workspace_bytes >= f16.workspace_bytes + 2 * pk.chunks
    assert pk.workspace_bytes <= f16.workspace_bytes + 2 * pk.chunks + 256
    assert pk.workspace_bytes % 256 == 0
    # with S = 8 and 32 the two planes cost 4 and 5 bits per element
    if S in (8, 32):
        bits = (pk.idx_bytes + pk.hnorm_bytes) * 8 / (pk.chunks * 4)
        assert bits == {8: 4.0, 32: 5.0}[S]


@pytest.mark.parametrize("seed,L,H,role,S", [(0, 1, 1, 0, 8), (0, 3, 5, 1, 32), (12345, 2, 2, 0, 1024),
                                             (2 ** 64 - 1, 1, 3, 1, 7)])
def test_codebook_matches_oracle_bit_for_bit(seed, L, H, role, S):
    a = K.hqmq_make_codebook(seed, L, H, role, S)
    b = O.make_codebook(seed, L, H, role, S)
    assert a.tobytes() == b.tobytes()


def test_library_codebook_is_on_the_double_binary16_grid():
    """hqmq_make_codebook returns every value as hi + lo with hi = fp16(q),
    lo = fp16(q - hi) (numpy's float16 rounding here, independent of both the
    library and the oracle), i.e. a value the kernels use unchanged."""
    q = K.hqmq_make_codebook(9, 3, 4, 1, 100).ravel()
    hi = q.astype(np.float16)
    lo = (q - hi.astype(np.float32)).astype(np.float16)
    assert np.array_equal(hi.astype(np.float32) + lo.astype(np.float32), q)
    # and not merely fp32: most values need the low part
    assert (lo != 0).mean() > 0.9


def test_exact_format_sizes_and_limits():
    """Exact-rate records: groups of 4 token rows whose word count is the
    oracle's; S not a power of two (24 S is then not 3 2^m) and paged pools
    are refused."""
    for S, D in ((8, 128), (32, 128), (1, 16), (1024, 256), (16, 64)):
        d = K.Desc.make(2, 3, 1001, D, S, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_EXACT)
        sz = K.hqmq_sizes(d)
        assert sz.group_rows == 4 and sz.group_words == O.exact_group_words(D // 4, S)
        assert sz.idx_bytes == 2 * 3 * 251 * sz.group_words * 4 and sz.hnorm_bytes == 0
    assert K.hqmq_sizes(K.Desc.make(1, 1, 4, 128, 8, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_EXACT)).group_words == 61
    assert K.hqmq_sizes(K.Desc.make(1, 1, 4, 128, 32, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_EXACT)).group_words == 77
    for S in (3, 13, 100):
        with pytest.raises(K.HQMQError) as e:
            K.hqmq_sizes(K.Desc.make(1, 1, 16, 128, S, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_EXACT))
        assert e.value.code == B.HQMQ_ENOTSUP
    with pytest.raises(K.HQMQError) as e:
        K.hqmq_paged_sizes(K.Desc.make(1, 1, 16, 128, 32, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_EXACT),
                           B.PagedDesc(4, 16, 8))
    assert e.value.code == B.HQMQ_ENOTSUP
    # the other formats report no groups
    assert K.hqmq_sizes(K.Desc.make(1, 1, 16, 128, 32)).group_words == 0


def test_codebook_validation():
    with pytest.raises(K.HQMQError):
        K.hqmq_make_codebook(0, 1, 1, 2, 8)
    with pytest.raises(K.HQMQError):
        K.hqmq_make_codebook(0, 1, 1, 0, 0)


# ---------------------------------------------------------------- attention
_CACHE = dict(layers=32, kv_heads=8, tokens=32 * 32768, head_dim=128, S=32, dtype=B.HQMQ_F16,
              med_batch_tokens=4096, med_C=3.0)


def _attn(**kw):
    a = dict(batch=32, group=4, layer=0, max_len=32768, scale=0.088)
    a.update(kw)
    return B.AttnDesc.make(**a)


def test_attn_plan_covers_every_token():
    d = K.Desc.make(**_CACHE)
    for batch, max_len in [(32, 32768), (1, 1), (3, 1000), (1, 200000), (64, 4096), (5, 0)]:
        s = B.hqmq_attn_sizes(d, _attn(batch=batch, max_len=max_len))
        assert s.split_tokens % 128 == 0 and s.split_tokens >= 128
        assert s.splits >= 1 and s.splits * s.split_tokens >= max_len
        assert (s.splits - 1) * s.split_tokens < max(max_len, 1)
        assert s.workspace_bytes == batch * 8 * 4 * s.splits * (128 + 2) * 4


@pytest.mark.parametrize("kw", [dict(group=0), dict(group=17), dict(layer=32), dict(layer=-1),
                                dict(batch=-1), dict(max_len=-1), dict(scale=float("inf")),
                                dict(scale=float("nan"))])
def test_attn_request_validation(kw):
    d = K.Desc.make(**_CACHE)
    with pytest.raises(K.HQMQError) as e:
        B.hqmq_attn_sizes(d, _attn(**kw))
    assert e.value.code == B.HQMQ_EINVAL


def test_attn_reserved_must_be_zero():
    d = K.Desc.make(**_CACHE)
    a = _attn()
    a.reserved = 1
    with pytest.raises(K.HQMQError):
        B.hqmq_attn_sizes(d, a)


@pytest.mark.parametrize("kw", [dict(dtype=B.HQMQ_F32), dict(head_dim=32), dict(head_dim=16)])
def test_attn_unsupported_caches(kw):
    c = dict(_CACHE)
    c.update(kw)
    with pytest.raises(K.HQMQError) as e:
        B.hqmq_attn_sizes(K.Desc.make(**c), _attn())
    assert e.value.code == B.HQMQ_ENOTSUP


def test_attend_rejects_before_enqueueing():
    """Validation fails before any HIP call: NULL buffers, short workspace."""
    d = K.Desc.make(**_CACHE)
    enc = B.Enc(16, 16, 16, 16, 16, 100, 16)
    L = B.lib()

    def call(q=16, start=16, length=16, out=16, ws=16, ws_bytes=1 << 30, a=None):
        return L.hqmq_attend(ctypes.byref(d), ctypes.byref(a or _attn()), ctypes.byref(enc), 16,
                             ctypes.byref(enc), 16, q, start, length, out, ws, ws_bytes, None)
    assert call(q=None) == B.HQMQ_EINVAL
    assert call(start=None) == B.HQMQ_EINVAL
    assert call(out=None) == B.HQMQ_EINVAL
    assert call(ws_bytes=100) == B.HQMQ_EINVAL
    assert call(q=18) == B.HQMQ_EINVAL          # misaligned query
    assert call(a=_attn(batch=0), q=None) == B.HQMQ_OK


# ---------------------------------------------------------------- paged pool
@pytest.mark.parametrize("nf", [0, 1])
def test_paged_sizes_follow_the_layout(nf):
    d = K.Desc.make(32, 8, 32, 128, 32, K.HQMQ_F16, 4096, 3.0, nf)
    p = K.PagedDesc(1000, 128, 256)
    s = K.hqmq_paged_sizes(d, p)
    W = 10
    rows = 32 * 8 * 1000 * 128
    assert s.idx_bytes == rows * W * 4
    assert s.hnorm_bytes == (rows * W * 4 if nf else rows * 32 * 2)
    assert s.side_count_bytes == 32 * 8 * 1000 * 4
    assert s.side_pos_bytes == 32 * 8 * 1000 * 256 * 4
    assert s.side_val_bytes == 32 * 8 * 1000 * 256 * 8
    # the call's records with a worst-case side list (16 outliers per token
    # of 32 chunks), plus the encode scratch
    c = K.hqmq_sizes(K.Desc.make(32, 8, 32, 128, 32, K.HQMQ_F16, 4096, 3.0))
    lo = c.idx_bytes + c.hnorm_bytes + c.offsets_bytes + 12 * c.max_outliers + c.workspace_bytes
    assert lo <= s.append_workspace_bytes <= lo + 8 * 256


@pytest.mark.parametrize("kw", [dict(page_tokens=48), dict(page_tokens=8), dict(page_tokens=0),
                                dict(num_pages=-1), dict(page_capacity=-1)])
def test_paged_desc_validation(kw):
    d = K.Desc.make(2, 2, 16, 128, 8, K.HQMQ_F16, 0, 3.0)
    p = dict(num_pages=10, page_tokens=64, page_capacity=16)
    p.update(kw)
    with pytest.raises(K.HQMQError) as e:
        K.hqmq_paged_sizes(d, K.PagedDesc(**p))
    assert e.value.code == B.HQMQ_EINVAL


def test_paged_calls_reject_before_enqueueing():
    lib = B.lib()
    d = K.Desc.make(1, 1, 4, 128, 8, K.HQMQ_F16, 4, 3.0)
    p = K.PagedDesc(4, 64, 8)
    pool = B.Pages()
    # null pool pointers, slots and workspace
    assert lib.hqmq_append(ctypes.byref(d), ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.c_void_p(16),
                           ctypes.byref(pool), None, None, 0, None) == B.HQMQ_EINVAL
    pool = B.Pages(16, 16, 16, 16, 16)
    assert lib.hqmq_append(ctypes.byref(d), ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.c_void_p(16),
                           ctypes.byref(pool), None, ctypes.c_void_p(256), 1 << 30, None) == B.HQMQ_EINVAL
    # workspace too small
    assert lib.hqmq_append(ctypes.byref(d), ctypes.byref(p), ctypes.c_void_p(16), ctypes.c_void_p(16),
                           ctypes.c_void_p(16), ctypes.byref(pool), None, ctypes.c_void_p(256), 64,
                           None) == B.HQMQ_EINVAL
    a = B.AttnDesc.make(1, 4, 0, 64, 0.1)
    # page-table stride 0
    assert lib.hqmq_attend_paged(ctypes.byref(d), ctypes.byref(p), ctypes.byref(a), ctypes.byref(pool),
                                 ctypes.c_void_p(16), ctypes.byref(pool), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                 ctypes.c_void_p(16), 0, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                 ctypes.c_void_p(256), 1 << 20, None) == B.HQMQ_EINVAL
    assert lib.hqmq_paged_clear(ctypes.byref(d), ctypes.byref(p), ctypes.byref(pool), None, 3,
                                None) == B.HQMQ_EINVAL


def _first_zero_keys(g0, g1, g2):
    """The search kernel's first-index choice on fp32 gaps (bit patterns):
    min3(g0, g1 | 1, med3(g2, 2, 3))."""
    b = [np.asarray(g, dtype=np.float32).view(np.uint32).astype(np.int64) for g in (g0, g1, g2)]
    k2 = np.clip(b[2], 2, 3)   # med3(x, 2, 3) = clamp to [2, 3]
    return np.minimum(np.minimum(b[0], b[1] | 1), k2)


def test_first_zero_gap_keys_give_the_first_zero_index():
    # Gaps max - value are +0 or multiples of 2^-48 of at least 2^-48 (scores
    # and transform components are multiples of 2^-48); as bit patterns the
    # keys are 0, 1, 2 for a zero gap and above 3 otherwise, so their minimum
    # is the index of the first zero gap, 3 when there is none.  Every zero /
    # nonzero pattern, with nonzero gaps from 2^-48 up to 2^40.
    rng = np.random.default_rng(7)
    n = 4096
    for pat in range(8):
        gaps = []
        for i in range(3):
            mag = np.ldexp(rng.integers(1, 1 << 20, n).astype(np.float64), rng.integers(-48, 21, n))
            mag = np.maximum(mag, 2.0 ** -48).astype(np.float32)
            gaps.append(np.where((pat >> i) & 1, np.float32(0.0), mag))
        want = np.where(gaps[0] == 0, 0, np.where(gaps[1] == 0, 1, np.where(gaps[2] == 0, 2, 3)))
        assert np.array_equal(_first_zero_keys(*gaps), want), pat
    # the smallest nonzero gap is far above the keys' range
    assert _first_zero_keys(np.float32(2.0 ** -48), np.float32(2.0 ** -48), np.float32(2.0 ** -48)) == 3
