"""Drive one encode + decode through the C ABI on the GPU and compare chosen
(layer, head) slices or batches with the oracle.  Used by the GPU tests,
``__graft_entry__.smoke()`` and the benchmark's sampled parity check."""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_quantization_hqmq_amd as K
import synth
from tests import parity as P


def desc_for(w: synth.Workload, tokens: int | None = None, norm_format: int = K.HQMQ_NORM_F16) -> K.Desc:
    return K.Desc.make(w.layers, w.heads, w.tokens if tokens is None else tokens, w.head_dim, w.S,
                       K.HQMQ_F32 if w.dtype == "f32" else K.HQMQ_F16, w.med_batch_tokens, w.med_C,
                       norm_format)


def codebook(w: synth.Workload, role: int, device="cuda"):
    host = K.hqmq_make_codebook(w.codebook_seed, w.layers, w.heads, role, w.S)
    return host, torch.from_numpy(host).to(device)


def run(desc: K.Desc, x: torch.Tensor, cb_dev: torch.Tensor, capacity=None):
    rec = K.encode(desc, x, cb_dev, capacity=capacity)
    y = K.decode(desc, rec, cb_dev)
    torch.cuda.synchronize()
    return rec, y


def compare(desc: K.Desc, x: torch.Tensor, cb_host: np.ndarray, rec, y: torch.Tensor,
            picks=None) -> P.Report:
    """picks: iterable of (layer, head, t0, T); default: every whole slice."""
    L, H, Tt, D = desc.shape
    B = int(desc.med_batch_tokens)
    nb = (Tt + min(B, Tt) - 1) // min(B, Tt) if (B > 0 and Tt > 0) else 0
    Bc = min(B, Tt) if B > 0 else 0
    if picks is None:
        picks = [(l, h, 0, Tt) for l in range(L) for h in range(H)]
    offs = rec.batch_offsets.cpu().numpy().view(np.uint64) if B > 0 else None
    rep = P.Report()
    for (l, h, t0, T) in picks:
        if T == 0:
            continue
        xs = x[l, h, t0:t0 + T].float().cpu().numpy()
        exact = desc.norm_format == K.HQMQ_NORM_EXACT
        if exact:   # the groups holding tokens [t0, t0 + T)
            words = rec.idx[l, h, t0 // 4:(t0 + T + 3) // 4].cpu().numpy()
            hn = None
        else:
            words = rec.idx[l, h, t0:t0 + T].cpu().numpy()
            hn = rec.hnorm[l, h, t0:t0 + T].cpu().numpy()
        ys = y[l, h, t0:t0 + T].cpu().numpy()
        pos = val = None
        if B > 0:
            sl = l * H + h
            b0, b1 = t0 // Bc, (t0 + T - 1) // Bc
            assert t0 % Bc == 0 and (t0 + T == Tt or (t0 + T) % Bc == 0), "picks must be whole batches"
            e0, e1 = int(offs[sl * nb + b0]), int(offs[sl * nb + b1 + 1])
            pos = rec.out_pos[e0:e1].cpu().numpy()
            val = rec.out_val[e0:e1].cpu().numpy()
        r = P.compare_slice(xs, cb_host[l, h], t0, Bc, float(desc.med_C), words, hn, pos, val, ys,
                            int(desc.S), desc.dtype == K.HQMQ_F32, desc.norm_format == K.HQMQ_NORM_PACKED,
                            exact)
        rep.merge(r)
    return rep
