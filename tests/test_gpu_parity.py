"""GPU parity: the HIP path (through the C ABI) against the oracle.

Small shapes are compared element by element on every chunk; they span
several encode tiles / decode blocks and end on a ragged tail (token counts
that are not multiples of the tile, Med3x batches with a partial last batch),
and cover both kernel families (S <= 32 register codebooks, larger S from
LDS), fp16 and fp32 inputs and every supported head_dim.
"""
import numpy as np
import pytest
import torch

import kv_cache_quantization_hqmq_amd as K
import oracle as O
import synth
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


def _check(desc, x, cb_host, cb_dev, capacity=None, picks=None):
    print(f"case {tuple(desc.shape)} S={desc.S} dtype={desc.dtype} B={desc.med_batch_tokens}", flush=True)
    rec, y = G.run(desc, x, cb_dev, capacity)
    rep = G.compare(desc, x, cb_host, rec, y, picks)
    print(dict(rep), flush=True)
    return rep, rec, y


def test_workload1_full():
    """Single-head fp32 K, 4096 x 128, S = 8, Med3x off: every chunk."""
    w = synth.WORKLOADS[1]
    x = synth.generate(w, 0, "cuda")
    cb_host, cb = G.codebook(w, 0)
    rep, _, _ = _check(G.desc_for(w), x, cb_host, cb)
    assert rep["chunks"] == w.chunks_per_role


CASES = [
    # (layers, heads, tokens, head_dim, S, dtype, med_batch_tokens)
    (2, 3, 1000, 128, 8, "f16", 0),
    (2, 3, 1501, 128, 32, "f16", 512),
    (1, 2, 777, 64, 13, "f16", 256),
    (1, 2, 333, 256, 1, "f32", 100),
    (2, 1, 129, 16, 40, "f16", 64),
    (1, 3, 64, 32, 100, "f32", 0),
    (1, 1, 97, 128, 1024, "f16", 32),
    (1, 1, 4100, 128, 32, "f32", 4096),
    (3, 2, 2051, 128, 8, "f16", 1024),
    # batches above 131072 chunks take the two-pass Med3x select
    (1, 1, 4200, 256, 32, "f16", 2100),
]


@pytest.mark.parametrize("L,H,T,D,S,dt,B", CASES)
def test_small_shapes_every_chunk(L, H, T, D, S, dt, B):
    dtype = torch.float16 if dt == "f16" else torch.float32
    x = _x((L, H, T, D), dtype, seed=L * 1000 + T + S)
    if B > 0:
        # outlier structure: a few hot channels and token spikes
        x[:, :, :, 5] *= 40
        x[:, :, ::97, :] *= 9
    cb_host, cb = _cb(L, H, S)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F32 if dt == "f32" else K.HQMQ_F16, B, 3.0)
    rep, rec, _ = _check(desc, x, cb_host, cb)
    if B > 0:
        assert rep["outliers"] > 0


# packed norm format: code widths b = 5 (exponent-only compact codes) to
# b = 15 (the binary16 pattern itself), with and without Med3x flags
PACKED_CASES = [
    (2, 3, 1000, 128, 8, "f16", 0),
    (2, 3, 1501, 128, 32, "f16", 512),
    (1, 2, 333, 256, 1, "f32", 100),
    (2, 1, 129, 16, 40, "f16", 64),
    (1, 1, 97, 128, 1024, "f16", 32),
    (1, 2, 777, 64, 13, "f16", 0),
]


@pytest.mark.parametrize("L,H,T,D,S,dt,B", PACKED_CASES)
def test_packed_norms_every_chunk(L, H, T, D, S, dt, B):
    """Every compact norm code and packed word against the oracle, decoded
    values from the half-norms the codes stand for; index codes and the side
    list are those of the binary16-format encode of the same input."""
    dtype = torch.float16 if dt == "f16" else torch.float32
    x = _x((L, H, T, D), dtype, seed=L * 1000 + T + S + 7)
    if B > 0:
        x[:, :, :, 5] *= 40
        x[:, :, ::97, :] *= 9
    cb_host, cb = _cb(L, H, S)
    f = K.HQMQ_F32 if dt == "f32" else K.HQMQ_F16
    desc = K.Desc.make(L, H, T, D, S, f, B, 3.0, K.HQMQ_NORM_PACKED)
    rep, rec, _ = _check(desc, x, cb_host, cb)
    ref, _ = G.run(K.Desc.make(L, H, T, D, S, f, B, 3.0), x, cb)
    assert torch.equal(rec.idx, ref.idx)
    assert rec.n_outliers == ref.n_outliers
    if B > 0:
        n = int(rec.n_outliers)
        assert n > 0
        assert torch.equal(rec.batch_offsets, ref.batch_offsets)
        assert torch.equal(rec.out_pos[:n], ref.out_pos[:n]) and torch.equal(rec.out_val[:n], ref.out_val[:n])


@pytest.mark.parametrize("S", [1, 8, 32])
def test_packed_norm_extremes(S):
    """Chunk norms from zero through binary16 subnormals to the top of the
    range (rounded up past the narrower format's largest value: capped), and
    values on the exact rounding ties of the compact code."""
    T, D = 256, 128
    cpt = D // 4
    rng = np.random.default_rng(S)
    # one nonzero component per chunk: the half-norm is |x0| / 2 exactly
    mag = np.ldexp(rng.uniform(1, 2, T * cpt), rng.integers(-24, 17, T * cpt))
    mag[:64] = 0.0
    mag[64:72] = [65504, 65504, 65472, 65440, 65376, 2.0 ** -24, 2.0 ** -23, 3 * 2.0 ** -24]
    b = O.code_bits(S)
    sh = 15 - b
    if sh > 0:
        # binary16 patterns halfway between two compact codes (x0 = 2 h16)
        pat = (rng.integers(1, 30 << 10, 200) >> sh << sh) + (1 << (sh - 1))
        mag[100:300] = 2.0 * pat.astype(np.uint16).view(np.float16).astype(np.float64)
    x = np.zeros((T * cpt, 4), np.float32)
    x[:, 0] = np.minimum(mag, 65504.0) * rng.choice([-1.0, 1.0], T * cpt)
    x[72:76] = 65504.0    # half-norm 65504: above the largest compact value for b < 15
    xt = torch.from_numpy(x.reshape(1, 1, T, D)).cuda()
    cb_host, cb = _cb(1, 1, S)
    for B in (0, 64):
        desc = K.Desc.make(1, 1, T, D, S, K.HQMQ_F32, B, 3.0, K.HQMQ_NORM_PACKED)
        _check(desc, xt, cb_host, cb)


def test_med3_many_chunks_at_the_threshold():
    """Two batches whose chunks have norm 1 except thousands at exactly C = 3
    times that norm or one binary16 step above or below it (and a few large
    outliers): the threshold code is crowded, so the single-pass select's
    list of undecided codes overflows in the first batch (6000 of them) and
    not in the second (1000); strict > leaves the chunks exactly at the
    threshold in the bulk."""
    T, D, B = 8192, 128, 4096
    cpt = D // 4
    x = np.full((T * cpt, 4), 0.5, np.float16)
    rng = np.random.default_rng(9)
    three_half = np.float16(1.5)
    vals = np.array([three_half, np.nextafter(three_half, np.float16(2)),
                     np.nextafter(three_half, np.float16(1))], np.float16)
    for b, m in ((0, 6000), (1, 1000)):
        idx = b * B * cpt + rng.choice(B * cpt, size=m, replace=False)
        x[idx] = vals[rng.integers(3, size=m)][:, None]
        big = b * B * cpt + rng.choice(B * cpt, size=50, replace=False)
        x[big] = np.float16(15.0)
    xt = torch.from_numpy(x.reshape(1, 1, T, D)).cuda()
    cb_host, cb = _cb(1, 1, 32)
    desc = K.Desc.make(1, 1, T, D, 32, K.HQMQ_F16, B, 3.0)
    rep, rec, _ = _check(desc, xt, cb_host, cb)
    assert rep["outliers"] > 0


def test_med3_crowded_median_bin():
    """One 131072-chunk batch whose median's code is shared by 2650 chunks at
    random positions (norm 1; 64000 chunks of norm 0.5 below them, the rest of
    norm 2 and 40 of norm 10 above): the single-pass select lists about 330
    loads per wave, more than it keeps in LDS (319), so some of their bytes are
    read again from memory, and the exact median is ranked among 2650 equal
    values."""
    T, D, B = 4096, 128, 4096
    n = T * D // 4
    rng = np.random.default_rng(17)
    x = np.full((n, 4), 1.0, np.float16)                  # norm 2
    idx = rng.permutation(n)
    x[idx[:64000]] = np.float16(0.25)                      # norm 0.5
    x[idx[64000:66650]] = np.float16(0.5)                  # norm 1: the median's code
    x[idx[66650:66690]] = np.float16(5.0)                  # norm 10 > 3 x 1: outliers
    xt = torch.from_numpy(x.reshape(1, 1, T, D)).cuda()
    cb_host, cb = _cb(1, 1, 32)
    desc = K.Desc.make(1, 1, T, D, 32, K.HQMQ_F16, B, 3.0)
    rep, rec, _ = _check(desc, xt, cb_host, cb)
    assert rep["outliers"] == 40


def test_med3_multiplier_below_one():
    """C = 0.5 on the crowded-median batch: the threshold s2 > 0.25 med puts
    the threshold code below the median's bin, so the single-pass select
    flags every code of that bin during its pass, and loads it visits again
    from memory (more than the 319 per wave it keeps in LDS) carry the flag;
    the median must still be ranked among the 2650 chunks of norm 1.  Every
    chunk of norm >= 1 is an outlier (67072, more than half the batch); the
    64000 chunks of norm 0.5 sit exactly at the threshold (s2 = 0.25 med) and
    stay in the bulk (strict >), decided by the pass over the whole batch
    since they overflow the undecided list."""
    T, D, B = 4096, 128, 4096
    n = T * D // 4
    rng = np.random.default_rng(17)
    x = np.full((n, 4), 1.0, np.float16)
    idx = rng.permutation(n)
    x[idx[:64000]] = np.float16(0.25)
    x[idx[64000:66650]] = np.float16(0.5)
    x[idx[66650:66690]] = np.float16(5.0)
    xt = torch.from_numpy(x.reshape(1, 1, T, D)).cuda()
    cb_host, cb = _cb(1, 1, 32)
    desc = K.Desc.make(1, 1, T, D, 32, K.HQMQ_F16, B, 0.5)
    assert K.hqmq_sizes(desc).max_outliers == n
    rep, rec, _ = _check(desc, xt, cb_host, cb)
    assert rep["outliers"] == n - 64000


@pytest.mark.parametrize("C", [0.5, 0.99, 1.0, 1.7])
def test_med3_other_multipliers_random(C):
    """Random heavy-tailed data with Med3x multipliers around 1 (binary16 and
    packed norms): outlier sets, codes and decoded values against the oracle."""
    L, H, T, D = 1, 2, 4100, 128
    x = _x((L, H, T, D), torch.float16, seed=int(C * 1000))
    x[:, :, :, 9] *= 30
    cb_host, cb = _cb(L, H, 32)
    for nf in (K.HQMQ_NORM_F16, K.HQMQ_NORM_PACKED):
        desc = K.Desc.make(L, H, T, D, 32, K.HQMQ_F16, 4096, C, nf)
        rep, _, _ = _check(desc, x, cb_host, cb)
        assert rep["outliers"] > 0


@pytest.mark.parametrize("S", [8, 13, 32, 40])
def test_repeated_codewords_take_the_first(S):
    """Codebooks whose entries repeat, as copies or negated copies (q and -q
    give the same 24 scores, 2T holding -1), before and after their source:
    every chunk whose best codeword repeats has exact score ties across s,
    among them ties between the two halves of the codebook that the fp16
    search scores in different lanes.  The smallest s wins, as in the
    oracle; zero chunks take s = 0."""
    L, H, T, D = 1, 2, 600, 64
    x = _x((L, H, T, D), torch.float16, seed=90 + S)
    x[:, :, ::37, :] = 0
    base, _ = _cb(L, H, S, seed=9)
    cb_host = base.copy()
    rng = np.random.default_rng(S)
    for s in range(S):
        if rng.random() < 0.6:
            src = base[:, :, rng.integers(0, S), :]
            cb_host[:, :, s, :] = -src if rng.random() < 0.3 else src
    assert len({tuple(v) for v in cb_host[0, 0]}) < S
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, 0, 3.0)
    _check(desc, x, cb_host, torch.from_numpy(cb_host).cuda())


@pytest.mark.parametrize("S", [32, 13])
def test_search_occupancy_cap_changes_no_output(S):
    """hqmq_set_search_blocks_per_cu only limits how many search blocks share
    a CU (the blocks reserve LDS they do not use): records, side list and
    decoded values are bit-identical at every cap."""
    L, H, T, D = 2, 2, 1500, 128
    x = _x((L, H, T, D), torch.float16, seed=31 + S)
    x[:, :, :, 7] *= 30
    cb_host, cb = _cb(L, H, S)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, 512, 3.0)

    def run():
        rec, y = G.run(desc, x, cb)
        torch.cuda.synchronize()
        n = rec.n_outliers
        return [t.cpu() for t in (rec.idx, rec.hnorm, rec.out_pos[:n], rec.out_val[:n], y)]

    ref = run()
    try:
        for cap in (7, 3, 1):
            K.hqmq_set_search_blocks_per_cu(cap)
            got = run()
            for a, b in zip(ref, got):
                assert torch.equal(a, b), cap
    finally:
        K.hqmq_set_search_blocks_per_cu(0)
    G.compare(desc, x, cb_host, *G.run(desc, x, cb))


def test_off_grid_codebook_encodes_like_its_rounded_copy():
    """The kernels use every codebook value on the double-binary16 grid
    (hi + lo binary16 parts): a codebook off the grid gives bit-identical
    records, decoded values and attention outputs to its rounded copy."""
    L, H, T, D, S = 2, 2, 1500, 128, 32
    x = _x((L, H, T, D), torch.float16, seed=77)
    x[:, :, :, 3] *= 25
    base = K.hqmq_make_codebook(5, L, H, 0, S)
    rng = np.random.default_rng(5)
    # nudge every value by a few fp32 ulps (off the 22-bit grid)
    off = (base * (1 + rng.integers(-6, 7, base.shape) * 2.0 ** -23)).astype(np.float32)
    assert (off != base).mean() > 0.5
    rounded = np.vectorize(O.codebook_value)(off).astype(np.float32)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, 512, 3.0)
    q = _x((1, H * 2, D), torch.float16, seed=78)
    st = torch.zeros(1, dtype=torch.int64, device="cuda")
    ln = torch.full((1,), T, dtype=torch.int32, device="cuda")
    outs = []
    for cb_host in (off, rounded):
        cb = torch.from_numpy(cb_host).cuda()
        rec, y = G.run(desc, x, cb)
        att = K.attend(desc, 1, rec, cb, rec, cb, q, st, ln, T)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (rec.idx, rec.hnorm, rec.out_pos[:rec.n_outliers],
                                        rec.out_val[:rec.n_outliers], y, att)])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    # and the records are the oracle's for the rounded codebook
    rec, y = G.run(desc, x, torch.from_numpy(off).cuda())
    G.compare(desc, x, rounded, rec, y)


def test_med3_select_writes_stay_inside_each_batch():
    """Head dim 16 (4 chunks per token row) and batches of 3 tokens: every
    batch ends inside a group of 8 code loads of the select, and each holds an
    outlier, so a group with a flag is only partly inside its batch.  The
    half-norm plane of the last slice is followed by sentinel chunks that must
    survive the encode (a write past a batch's end lands there for the last
    batch), and the records match the oracle."""
    L, H, T, D, S, B = 2, 1, 37, 16, 8, 3
    cpt = D // 4
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((L, H, T, cpt, 4)) * 0.1).astype(np.float16)
    for l in range(L):
        for t0 in range(0, T, B):
            x[l, 0, t0, rng.integers(cpt)] = np.float16(4.0)   # one outlier per batch
    xt = torch.from_numpy(x.reshape(L, H, T, D)).cuda()
    cb_host, cb = _cb(L, H, S)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, B, 3.0)
    rec = K.allocate_records(desc)
    n = L * H * T * cpt
    guard = torch.full((n + 256,), 0x5A5A, dtype=torch.int16, device="cuda")
    rec.hnorm = guard[:n].view(L, H, T, cpt)
    rec.c.hnorm = guard.data_ptr()
    ws = K.workspace(desc)
    K.hqmq_encode(desc, xt, cb, rec, ws, torch.cuda.current_stream().cuda_stream)
    n_out = K.hqmq_encode_result(rec, torch.cuda.current_stream().cuda_stream)
    y = K.decode(desc, rec, cb)
    torch.cuda.synchronize()
    assert torch.all(guard[n:] == 0x5A5A), "the select wrote past the last batch"
    rep = G.compare(desc, xt, cb_host, rec, y)
    print(dict(rep), flush=True)
    assert n_out >= L * ((T + B - 1) // B)


def _guarded(t: torch.Tensor, pad_bytes: int = 4096):
    """A tensor of t's shape and dtype at the front of a larger buffer whose
    tail holds a byte pattern: writes past the tensor's end change the tail."""
    nbytes = t.numel() * t.element_size()
    buf = torch.full((nbytes + pad_bytes,), 0xA5, dtype=torch.uint8, device=t.device)
    return buf[:nbytes].view(t.dtype).view(t.shape), buf, nbytes


@pytest.mark.parametrize("L,H,T,D,S,dt,B,norm", [
    (2, 3, 41, 16, 8, "f16", 3, "f16"),
    (1, 2, 77, 64, 40, "f16", 5, "packed"),
    (2, 1, 33, 16, 100, "f32", 7, "f16"),
    (1, 1, 130, 128, 32, "f16", 64, "packed"),
    (2, 3, 43, 16, 8, "f16", 4, "exact"),
    (1, 2, 131, 128, 32, "f32", 64, "exact"),
    (1, 1, 70, 256, 1024, "f16", 16, "exact"),
])
def test_outputs_stay_inside_their_buffers(L, H, T, D, S, dt, B, norm):
    """Every record plane, the side list, its offsets and the decoded tensor
    sit at the front of buffers with a patterned tail: after encode and decode
    on ragged shapes (small head dims, partial batches and token rows, packed
    and binary16 norms, fp16 and fp32 input) every tail is unchanged and the
    result matches the oracle."""
    dtype = torch.float16 if dt == "f16" else torch.float32
    x = _x((L, H, T, D), dtype, seed=T * 7 + S)
    x[:, :, :, 5] *= 40                      # hot channel: outliers in every batch
    cb_host, cb = _cb(L, H, S)
    nf = {"packed": K.HQMQ_NORM_PACKED, "exact": K.HQMQ_NORM_EXACT}.get(norm, K.HQMQ_NORM_F16)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F32 if dt == "f32" else K.HQMQ_F16, B, 3.0, nf)
    rec = K.allocate_records(desc, K.hqmq_sizes(desc).max_outliers)
    guards = []
    for name, field in (("idx", "idx"), ("hnorm", "hnorm"), ("batch_offsets", "batch_offsets"),
                        ("out_pos", "out_pos"), ("out_val", "out_val")):
        t = getattr(rec, name)
        if t is None:   # the exact format has no norm plane
            continue
        g, buf, nb = _guarded(t)
        setattr(rec, name, g)
        setattr(rec.c, field, buf.data_ptr())
        guards.append((name, buf, nb))
    ws = K.workspace(desc)
    st = torch.cuda.current_stream().cuda_stream
    K.hqmq_encode(desc, x, cb, rec, ws, st)
    rec.n_outliers = K.hqmq_encode_result(rec, st)
    y, ybuf, ynb = _guarded(torch.empty(desc.shape, dtype=dtype, device="cuda"))
    K.hqmq_decode(desc, rec, cb, y, st)
    torch.cuda.synchronize()
    for name, buf, nb in guards + [("y", ybuf, ynb)]:
        assert torch.all(buf[nb:] == 0xA5), f"{name}: written past its end"
    rep = G.compare(desc, x, cb_host, rec, y)
    print(dict(rep), flush=True)
    assert rep["outliers"] > 0


def test_empty_inputs():
    cb_host, cb = _cb(1, 1, 8)
    for T in (0,):
        desc = K.Desc.make(1, 1, T, 128, 8, K.HQMQ_F16, 64, 3.0)
        x = torch.empty((1, 1, T, 128), dtype=torch.float16, device="cuda")
        rec, y = G.run(desc, x, cb)
        assert rec.n_outliers == 0
        assert int(rec.batch_offsets[0]) == 0
    desc = K.Desc.make(0, 4, 16, 128, 8, K.HQMQ_F16, 0, 3.0)
    x = torch.empty((0, 4, 16, 128), dtype=torch.float16, device="cuda")
    rec, y = G.run(desc, x, cb)
    assert y.numel() == 0


def test_single_token_and_tiny_batches():
    for T, B in ((1, 1), (2, 1), (3, 2), (65, 64)):
        x = _x((1, 2, T, 128), torch.float16, seed=T)
        cb_host, cb = _cb(1, 2, 32)
        desc = K.Desc.make(1, 2, T, 128, 32, K.HQMQ_F16, B, 3.0)
        _check(desc, x, cb_host, cb)


@pytest.mark.parametrize("case", ["inflated_rows", "some_rows_inflated", "crowded_outliers"])
def test_med3_uneven_batches(case):
    """Med3x batches of 32768 chunks whose outliers are spread unevenly: the
    first 8 token rows of every 256 x 100 (a few huge rows, and the hot
    channel's outliers everywhere else), the same in every third 256-row block
    only, or the first 26 channels x 30 (22% of the chunks are outliers).  The
    side list, flags and codes must be bit-exact with the oracle."""
    L, H, T, D, S, B = 1, 2, 3000, 128, 32, 1024
    x = _x((L, H, T, D), torch.float16, seed=17)
    x[:, :, :, 5] *= 40
    rows = torch.arange(T, device="cuda")
    first_rows = (rows % 256) < 8
    if case == "inflated_rows":
        x[:, :, first_rows, :] *= 100
    elif case == "some_rows_inflated":
        x[:, :, first_rows & ((rows // 256) % 3 == 1), :] *= 100
    else:
        x[:, :, :, :26] *= 30
    cb_host, cb = _cb(L, H, S)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, B, 3.0)
    rep, _, _ = _check(desc, x, cb_host, cb)
    assert rep["outliers"] > 0


def test_zero_and_degenerate_batches():
    """All-zero slice (median 0, no outlier), half-zero batch (median 0: every
    nonzero chunk is an outlier), fp16 extremes."""
    L, H, T, D, S = 1, 3, 256, 128, 32
    x = _x((L, H, T, D), torch.float16, seed=5)
    x[0, 0] = 0
    x[0, 1, : T // 2 + 1] = 0
    x[0, 2, 7, :8] = 65504
    x[0, 2, 9, 4:8] = -65504
    x[0, 2, 11, :4] = torch.tensor([6e-8, 0, 0, 0], dtype=torch.float16)
    cb_host, cb = _cb(L, H, S)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, T, 3.0)
    rep, rec, y = _check(desc, x, cb_host, cb)
    offs = rec.batch_offsets.cpu().numpy()
    assert offs[1] - offs[0] == 0                       # all-zero slice
    assert offs[2] - offs[1] == int((x[0, 1].float().reshape(-1, 4).abs().sum(1) > 0).sum())
    assert torch.all(y[0, 0] == 0)


def test_codeword_inputs_round_trip():
    """x = rho * codeword (fp32): the codeword maps to itself and decodes back
    within the fp16 rounding of the norm."""
    S, T, D = 32, 64, 128
    cb_host, cb = _cb(1, 1, S)
    rng = np.random.default_rng(3)
    cw = np.stack([O.codeword(cb_host[0, 0], k) for k in range(24 * S)])
    ks = rng.integers(0, 24 * S, T * D // 4)
    rho = rng.uniform(0.5, 20, len(ks))
    xh = (rho[:, None] * cw[ks]).astype(np.float32).reshape(1, 1, T, D)
    x = torch.from_numpy(xh).cuda()
    desc = K.Desc.make(1, 1, T, D, S, K.HQMQ_F32, 0, 3.0)
    rep, rec, y = _check(desc, x, cb_host, cb)
    from tests.parity import unpack_words
    codes = unpack_words(rec.idx.cpu().numpy().view(np.uint32)[0, 0], D // 4, 10).reshape(-1)
    assert np.array_equal(codes, ks)
    err = np.abs(y.cpu().numpy() - xh).reshape(-1, 4).max(1)
    assert np.all(err <= 2.0 ** -10 * rho)


def test_deep_hole_tie_takes_smallest_code():
    """S = 1, q = 1: u = (1,1,0,0)/sqrt2 ties six 2T vertices; smallest k wins
    (exact fp32 tie on the GPU too)."""
    q = np.zeros((1, 1, 1, 4), np.float32)
    q[..., 0] = 1
    x = torch.zeros((1, 1, 4, 16), dtype=torch.float32, device="cuda")
    x[0, 0, :, 0] = 1
    x[0, 0, :, 1] = 1
    desc = K.Desc.make(1, 1, 4, 16, 1, K.HQMQ_F32, 0, 3.0)
    rec, y = G.run(desc, x, torch.from_numpy(q).cuda())
    from tests.parity import unpack_words
    codes = unpack_words(rec.idx.cpu().numpy().view(np.uint32)[0, 0], 4, 5)
    assert codes[:, 0].tolist() == [0, 0, 0, 0]
    assert codes[:, 1:].tolist() == [[0] * 3] * 4       # zero chunks


def test_deterministic():
    x = _x((2, 2, 3000, 128), torch.float16, seed=9)
    x[:, :, :, 3] *= 50
    cb_host, cb = _cb(2, 2, 32)
    desc = K.Desc.make(2, 2, 3000, 128, 32, K.HQMQ_F16, 1024, 3.0)
    a, ya = G.run(desc, x, cb)
    b, yb = G.run(desc, x, cb)
    for f in ("idx", "hnorm", "batch_offsets"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    n = int(a.n_outliers)
    assert n > 0
    assert torch.equal(a.out_pos[:n], b.out_pos[:n]) and torch.equal(a.out_val[:n], b.out_val[:n])
    assert torch.equal(ya, yb)


def test_capacity_overflow_reports_needed_count():
    x = _x((1, 2, 2048, 128), torch.float16, seed=11)
    x[:, :, :, 7] *= 60
    cb_host, cb = _cb(1, 2, 8)
    desc = K.Desc.make(1, 2, 2048, 128, 8, K.HQMQ_F16, 512, 3.0)
    ws = K.workspace(desc)
    rec = K.allocate_records(desc, capacity=10)
    K.hqmq_encode(desc, x, cb, rec, ws)
    with pytest.raises(K.CapacityError) as ei:
        K.hqmq_encode_result(rec)
    need = ei.value.needed
    assert need > 10
    rec2, y2 = G.run(desc, x, cb, capacity=need)
    assert rec2.n_outliers == need
    G.compare(desc, x, cb_host, rec2, y2)


def test_capacity_overflow_decodes_dropped_chunks_to_bulk_values():
    """With the side list cut at the capacity, the outlier chunks whose entries
    were dropped decode to the bulk value of their record (nearest codeword
    times the half-norm), kept entries exactly, and attention reads the same
    values as the decoder."""
    import math
    from tests import attend_cases as A
    x = _x((1, 2, 2048, 128), torch.float16, seed=12)
    x[:, :, :, 7] *= 60
    cb_host, cb = _cb(1, 2, 32)
    desc = K.Desc.make(1, 2, 2048, 128, 32, K.HQMQ_F16, 512, 3.0)
    cap = 700
    rec = K.allocate_records(desc, capacity=cap)
    K.hqmq_encode(desc, x, cb, rec, K.workspace(desc))
    with pytest.raises(K.CapacityError) as ei:
        K.hqmq_encode_result(rec)
    assert ei.value.needed > cap
    y = K.decode(desc, rec, cb)
    torch.cuda.synchronize()
    offs = rec.batch_offsets.cpu().numpy().view(np.uint64)
    pos = rec.out_pos[:cap].cpu().numpy().view(np.uint32)
    nb = 4
    b = O.code_bits(32)
    dropped_any = 0
    for h in range(2):
        codes = P_unpack(rec.idx[0, h].cpu().numpy().view(np.uint32), 32, b).reshape(-1)
        hn = rec.hnorm[0, h].cpu().numpy().view(np.uint16).reshape(-1)
        flagged = (hn & 0x8000) != 0
        kept = np.zeros(hn.shape, bool)
        e0, e1 = min(int(offs[h * nb]), cap), min(int(offs[(h + 1) * nb]), cap)
        kept[pos[e0:e1]] = True
        dropped = flagged & ~kept
        dropped_any += int(dropped.sum())
        bulk = A.f16_values(O.decode_range(codes, hn & 0x7FFF, 2048, 128, cb_host[0, h])).reshape(-1, 4)
        yg = y[0, h].float().cpu().numpy().astype(np.float64).reshape(-1, 4)
        rhat = 2.0 * (hn & 0x7FFF).view(np.float16).astype(np.float64)
        err = np.abs(yg - bulk).max(axis=1)
        lim = np.maximum(1e-3 * rhat, 2.0 ** -24)
        assert np.all(err[~kept] <= lim[~kept])
        xs = x[0, h].float().cpu().numpy().reshape(-1, 4).astype(np.float16).astype(np.float64)
        np.testing.assert_array_equal(yg[kept], xs[kept])
    assert dropped_any > 0
    # attention over the same records reads the decoder's values
    q = A.make_queries(1, 8, 128, 5)
    out = K.attend(desc, 0, rec, cb, rec, cb, q, torch.zeros(1, dtype=torch.int64, device="cuda"),
                   torch.full((1,), 2048, dtype=torch.int32, device="cuda"), 2048)
    torch.cuda.synchronize()
    qn = q.float().cpu().numpy().astype(np.float64)
    for h in range(2):
        v = y[0, h].float().cpu().numpy().astype(np.float64)
        ref = O.attend(v, v, qn[0, 4 * h:4 * h + 4], 1.0 / math.sqrt(128))
        assert A.compare_out(out.cpu().numpy()[0, 4 * h:4 * h + 4], ref, v) <= 1.0


def P_unpack(words, cpt, b):
    from tests.parity import unpack_words
    return unpack_words(words, cpt, b)


def test_invalid_arguments_enqueue_nothing():
    x = _x((1, 1, 64, 128), torch.float16, seed=1)
    cb_host, cb = _cb(1, 1, 8)
    desc = K.Desc.make(1, 1, 64, 128, 8, K.HQMQ_F16, 16, 3.0)
    rec = K.allocate_records(desc)
    with pytest.raises(K.HQMQError):
        K.hqmq_encode(desc, x, cb, rec, None)          # workspace missing
    with pytest.raises(K.HQMQError):
        K.hqmq_encode(desc, x[..., 1:], cb, rec, K.workspace(desc))   # misaligned input
    bad = K.Desc.make(1, 1, 64, 96, 8, K.HQMQ_F16, 16, 3.0)
    with pytest.raises(K.HQMQError):
        K.hqmq_encode(bad, x, cb, rec, K.workspace(desc))
