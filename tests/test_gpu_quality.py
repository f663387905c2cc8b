"""GPU quality checks on synthetic inputs (the full report is
`python3 bench.py --quality`): the covering trend of the random
multiplicative codebook (Prop. 3.1, gist.science/nl "Methodologie" 2: the
error falls as (24 S)^(-1/3); only the trend is checked, the constant is not
given) and the effect of Med3x on outlier-heavy K/V (gist.science/nl
"Methodologie" 3)."""
import math

import numpy as np
import pytest
import torch

import bench
import kv_cache_quantization_hqmq_amd as K
import synth

pytestmark = pytest.mark.gpu


def _roundtrip(w, x, role, S, B):
    desc = K.Desc.make(w.layers, w.heads, w.tokens, w.head_dim, S, K.HQMQ_F16, B, 3.0)
    cb = torch.from_numpy(K.hqmq_make_codebook(w.codebook_seed, w.layers, w.heads, role, S)).cuda()
    rec = K.encode(desc, x, cb)
    return K.decode(desc, rec, cb)


def test_covering_trend_against_codewords():
    w = synth.WORKLOADS[2].scaled(layers=2, heads=4, tokens=4096, dist="normal", data_seed=4411)
    x = synth.generate(w, 0, "cuda")
    Ss = (1, 4, 16, 64, 256)
    ang = [bench._errors(x, _roundtrip(w, x, 0, S, 0))["chunk_angle_deg"] for S in Ss]
    print(dict(zip(Ss, ang)), flush=True)
    assert all(a > b for a, b in zip(ang, ang[1:]))
    slope = np.polyfit(np.log([24 * S for S in Ss]), np.log(ang), 1)[0]
    assert -0.40 < slope < -0.26, slope


def test_med3_on_outlier_heavy_kv():
    w = synth.WORKLOADS[3].scaled(layers=2, heads=4, tokens=8192, data_seed=4412)
    xs = {r: synth.generate(w, r, "cuda") for r in (0, 1)}
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q = torch.randn((w.layers, w.heads, w.head_dim), generator=g, device="cuda").to(torch.float16)
    sc = 1.0 / math.sqrt(w.head_dim)
    res = {}
    for name, B in (("med3", 4096), ("off", 0)):
        ys = {r: _roundtrip(w, xs[r], r, 32, B) for r in (0, 1)}
        res[name] = (bench._errors(torch.cat([xs[0], xs[1]]), torch.cat([ys[0], ys[1]]))["rel_mse"],
                     bench._attention_error(xs[0], xs[1], ys[0], ys[1], q, sc))
    y4 = {r: bench._int_per_token(xs[r], 4) for r in (0, 1)}
    int4 = bench._attention_error(xs[0], xs[1], y4[0], y4[1], q, sc)
    print(res, "int4 attention", int4, flush=True)
    assert res["med3"][0] * 10 < res["off"][0]
    assert res["med3"][1] < res["off"][1] and res["med3"][1] < int4
