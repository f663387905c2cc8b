"""hqmq_attend_noalloc: the attention entry point that allocates nothing
(its split partials live in a library-owned per-GPU device array) must give
exactly hqmq_attend's outputs (the same kernels, so bit for bit), call after
call on the shared array, and must reject a request larger than that array
on the host."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_hqmq_amd as K
from kv_cache_quantization_hqmq_amd import hqmq as B

pytestmark = pytest.mark.gpu


def _cache(L, H, T, D, S, Bmed, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, Bmed, 3.0)
    recs, cbs = [], []
    for role in (0, 1):
        x = torch.randn((L, H, T, D), generator=g, device="cuda")
        x[..., 7] *= 30
        x = x.to(torch.float16)
        cb = torch.from_numpy(K.hqmq_make_codebook(11, L, H, role, S)).cuda()
        recs.append(K.encode(desc, x, cb))
        cbs.append(cb)
    return desc, recs, cbs


def _both(desc, layer, recs, cbs, batch, group, starts, lens, max_len, seed):
    D = int(desc.head_dim)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((batch, desc.kv_heads * group, D), generator=g, device="cuda").to(torch.float16)
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    a = K.AttnDesc.make(batch, group, layer, max_len, 1.0 / np.sqrt(D))
    ws = torch.empty((max(int(K.hqmq_attn_sizes(desc, a).workspace_bytes), 16),), dtype=torch.uint8,
                     device="cuda")
    ref = torch.full((batch, desc.kv_heads * group, D), float("nan"), device="cuda")
    out = torch.full_like(ref, float("nan"))
    K.hqmq_attend(desc, a, recs[0], cbs[0], recs[1], cbs[1], q, st, ln, ref, ws)
    B.hqmq_attend_noalloc(desc, a, recs[0], cbs[0], recs[1], cbs[1], q, st, ln, out)
    torch.cuda.synchronize()
    return ref.cpu(), out.cpu()


def test_noalloc_matches_the_workspace_call_twice_second_smaller():
    """Two calls in a row on the shared array: a larger one (12 sequences of
    up to 3000 tokens, GQA 4, several splits each) then a smaller one (3
    sequences, GQA 2, one of them empty): each equals hqmq_attend bit for
    bit, so the second call reads nothing the first one left."""
    print("case: noalloc vs workspace, two calls", flush=True)
    desc, recs, cbs = _cache(2, 4, 3000, 128, 32, 512, seed=5)
    rng = np.random.default_rng(5)
    starts = [int(s) for s in rng.integers(0, 1000, 12)]
    lens = [int(min(3000 - s, l)) for s, l in zip(starts, rng.integers(1, 2500, 12))]
    ref, out = _both(desc, 1, recs, cbs, 12, 4, starts, lens, max(lens), seed=6)
    assert torch.isfinite(ref).all()
    assert torch.equal(ref, out)
    ref2, out2 = _both(desc, 0, recs, cbs, 3, 2, [0, 100, 2999], [1500, 0, 1], 1500, seed=7)
    assert torch.equal(ref2, out2)
    assert torch.all(out2[1] == 0)


def test_noalloc_head_dim_64_packed_norms():
    print("case: noalloc head_dim 64", flush=True)
    L, H, T, D, S = 1, 2, 700, 64, 8
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    desc = K.Desc.make(L, H, T, D, S, K.HQMQ_F16, 0, 3.0, K.HQMQ_NORM_PACKED)
    recs, cbs = [], []
    for role in (0, 1):
        x = torch.randn((L, H, T, D), generator=g, device="cuda").to(torch.float16)
        cb = torch.from_numpy(K.hqmq_make_codebook(3, L, H, role, S)).cuda()
        recs.append(K.encode(desc, x, cb))
        cbs.append(cb)
    ref, out = _both(desc, 0, recs, cbs, 2, 8, [0, 33], [700, 600], 700, seed=10)
    assert torch.equal(ref, out)


def test_noalloc_rejects_requests_beyond_its_scratch():
    """A request whose partials would exceed the array is refused on the
    host with HQMQ_ENOTSUP (nothing is enqueued, so no buffers are needed)."""
    desc = K.Desc.make(1, 64, 1 << 20, 256, 32, K.HQMQ_F16, 0, 3.0)
    a = K.AttnDesc.make(256, 16, 0, 1 << 20, 0.0625)
    assert K.hqmq_attn_sizes(desc, a).workspace_bytes > B.HQMQ_ATTEND_SCRATCH_BYTES
    dummy = K.allocate_records(K.Desc.make(1, 64, 0, 256, 32, K.HQMQ_F16, 0, 3.0), device="cuda")
    with pytest.raises(K.HQMQError) as e:
        B.hqmq_attend_noalloc(desc, a, dummy, None, dummy, None, None, None, None, None)
    assert e.value.code == B.HQMQ_ENOTSUP
