"""GPU parity at the workloads' full sizes, on sampled outputs.

Each workload is encoded and decoded whole on the GPU through the C ABI (the
same calls and launch configuration the benchmark times); seeded samples of
whole (layer, head) token ranges or whole Med3x batches are then compared
with the oracle element by element (codes, half-norm codes and flags, side
list, decoded values).  Roles are run one at a time to bound memory.
"""
import numpy as np
import pytest
import torch

import kv_cache_quantization_hqmq_amd as K
import synth
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu


def _picks(w: synth.Workload, n: int, seed: int, span: int):
    """n seeded (layer, head, t0, T) picks: whole Med3x batches when Med3x is
    on, else token ranges of length span; always includes the last one."""
    rng = np.random.default_rng(seed)
    B = w.med_batch_tokens or span
    nb = -(-w.tokens // B)
    out = [(w.layers - 1, w.heads - 1, (nb - 1) * B, w.tokens - (nb - 1) * B)]
    for _ in range(n - 1):
        l, h, b = int(rng.integers(w.layers)), int(rng.integers(w.heads)), int(rng.integers(nb))
        out.append((l, h, b * B, min(B, w.tokens - b * B)))
    return out


def _run_role(w: synth.Workload, role: int, n_picks: int, span: int = 2048, norm_format: int = K.HQMQ_NORM_F16):
    print(f"workload {w.name} role {role} norm format {norm_format}: {synth.describe(w)}", flush=True)
    x = synth.generate(w, role, "cuda")
    cb_host, cb = G.codebook(w, role)
    d = G.desc_for(w, norm_format=norm_format)
    rec, y = G.run(d, x, cb)
    rep = G.compare(d, x, cb_host, rec, y, _picks(w, n_picks, 100 * w.wid + role, span))
    print(dict(rep), "outliers total", rec.n_outliers, flush=True)
    assert rep["code_mismatch"] <= rep["exempt"]
    del x, y, rec
    torch.cuda.empty_cache()
    return rep


@pytest.mark.parametrize("role", [0, 1])
def test_mistral7b_kv_32k_s8(role):
    _run_role(synth.WORKLOADS[2], role, n_picks=6)


@pytest.mark.parametrize("role", [0, 1])
def test_qwen_outlier_kv_32k_s32_med3(role):
    rep = _run_role(synth.WORKLOADS[3], role, n_picks=5)
    assert rep["outliers"] > 0


@pytest.mark.parametrize("role", [0, 1])
def test_llama3_70b_kv_128k_s32_med3(role):
    rep = _run_role(synth.WORKLOADS[4], role, n_picks=4)
    if role == 0:
        assert rep["outliers"] > 0


@pytest.mark.parametrize("role", [0, 1])
@pytest.mark.parametrize("norm_format", [K.HQMQ_NORM_PACKED, K.HQMQ_NORM_EXACT])
def test_llama3_70b_kv_128k_s32_med3_compact_norms(role, norm_format):
    """The packed and the exact-rate records of the whole 128k cache (their
    pack kernels and decoders at full size: the exact-rate decode takes one
    group of 4 rows per wave step here), sampled whole Med3x batches against
    the oracle."""
    rep = _run_role(synth.WORKLOADS[4], role, n_picks=3, norm_format=norm_format)
    if role == 0:
        assert rep["outliers"] > 0


@pytest.mark.parametrize("role", [0, 1])
def test_llama3_8b_decode_step_32x32k(role):
    """Decode-step workload: the 32-sequence x 32768-token cache (sequences
    stacked on the token axis of each (layer, head)) encoded with Med3x per
    4096 tokens, one decode step's appended tokens (one per sequence and
    layer) encoded as their own segment with the step as the Med3x batch,
    and the whole cache decoded."""
    w = synth.WORKLOADS[5]
    if True:
        print(f"decode-step cache role {role}", flush=True)
        x = synth.generate(w, role, "cuda")
        cb_host, cb = G.codebook(w, role)
        d = G.desc_for(w)
        rec = K.encode(d, x, cb)
        picks = _picks(w, 3, 500 + role, 2048)
        # keep the sampled inputs, then decode into the input's buffer
        xs = {p: x[p[0], p[1], p[2]:p[2] + p[3]].clone() for p in picks}
        K.decode(d, rec, cb, y=x)
        torch.cuda.synchronize()
        rep = _compare_picks(d, xs, cb_host, rec, x, picks)
        print(dict(rep), flush=True)
        assert rep["outliers"] > 0
        del x, rec
        torch.cuda.empty_cache()
        # the step's appended tokens: [layers, heads, 32 (one per sequence), 128]
        xa = synth.generate_append(w, role, step=0, device="cuda")
        da = K.Desc.make(w.layers, w.heads, w.append_tokens, w.head_dim, w.S, K.HQMQ_F16,
                         w.append_tokens, w.med_C)
        reca, ya = G.run(da, xa, cb)
        repa = G.compare(da, xa, cb_host, reca, ya)
        print("appended", dict(repa), flush=True)


def _compare_picks(d, xs, cb_host, rec, y, picks):
    """G.compare for inputs held per pick (the full input was overwritten)."""
    from tests import parity as P
    L, H, Tt, D = d.shape
    B = int(d.med_batch_tokens)
    Bc = min(B, Tt)
    nb = -(-Tt // Bc)
    offs = rec.batch_offsets.cpu().numpy().view(np.uint64)
    rep = P.Report()
    for (l, h, t0, T) in picks:
        sl = l * H + h
        b0, b1 = t0 // Bc, (t0 + T - 1) // Bc
        e0, e1 = int(offs[sl * nb + b0]), int(offs[sl * nb + b1 + 1])
        r = P.compare_slice(xs[(l, h, t0, T)].float().cpu().numpy(), cb_host[l, h], t0, Bc, float(d.med_C),
                            rec.idx[l, h, t0:t0 + T].cpu().numpy(), rec.hnorm[l, h, t0:t0 + T].cpu().numpy(),
                            rec.out_pos[e0:e1].cpu().numpy(), rec.out_val[e0:e1].cpu().numpy(),
                            y[l, h, t0:t0 + T].cpu().numpy(), int(d.S), False)
        rep.merge(r)
    return rep
