#!/usr/bin/env python3
"""HQMQ encode + decode throughput on one MI355X.

One step is one pass of the whole codec over the resident cache: for K and
for V, hqmq_encode (norm code, nearest of the 24 S codewords, Med3x median,
outlier side list) and hqmq_decode (gather-multiply plus outlier
re-insertion).  The default workload is the Llama-3-70B 128k-context cache
(80 layers x 8 KV heads x 131072 tokens x 128, K and V fp16, S = 32, Med3x
C = 3 per 4096-token batch): the pages' storage example and the largest
single-GPU configuration, and the one that exercises every step.

Prints one JSON line.  ``value`` counts chunks (4-element groups) per second,
each chunk encoded and decoded once per step.  ``roofline`` is the encode
search kernel, timed with HIP events recorded by the library around that
kernel on the launch stream, against the dense f16 peak of the matrix-core
instruction it issues (with the committed VALU counters beside it: the
epilogue on the vector ALUs is what binds it); ``roofline_decode`` is the
decode kernel against HBM bandwidth.  ``cpu_baseline`` is the plain C oracle
timed on a bounded sample of the same workload on this host.  By default the
line also carries the same step in the other norm formats (``formats``) and
the decode-step workload's figures (``decode_step``: attention read from the
records against decoding the whole cache each step).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HQMQ encode & decode chunks/s and GB/s (fp16 in) on 1 MI355X; % of roofline"
PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense f16 matrix cores
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 (vector and matrix)
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
NORM_FORMATS = {"f16": 0, "packed": 1, "exact": 2}   # hqmq_desc.norm_format
_CSRC = os.path.join(ROOT, "kv_cache_quantization_hqmq_amd", "csrc")
# the sources a committed counter summary was taken from (codec; attention)
KERNEL_SRC = [os.path.join(_CSRC, f) for f in ("hqmq_kernels.hip", "hqmq_search.hip", "hqmq_encode.h",
                                                "hqmq_device.h")]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_llama3-70b-kv-128k.json")
COUNTERS5_FILE = os.path.join(ROOT, "profiles", "counters_llama3-8b-decode-32x32k.json")
ATTEND_SRC = [os.path.join(_CSRC, f) for f in ("hqmq_attend.hip", "hqmq_device.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (events on an arbitrary
    stream; torch.cuda.Event only records on torch's current stream)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream: int):
        assert self.rt.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def ms(self, a, b) -> float:
        t = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return float(t.value)

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


def measure_ceilings(src, dst, stream: int, ev) -> dict:
    """This GPU's measured ceilings (context beside the published peaks):
    streaming read, write and copy over 4 GiB of device memory (src and dst:
    device tensors of at least that size, overwritten), non-packed fp32 FMA on
    the VALU, and the fp32 and f16 matrix cores.  Each figure is the median
    of 3 timed launches after one untimed."""
    import torch
    import kv_cache_quantization_hqmq_amd as K
    nbytes = 4 << 30
    assert src.numel() * src.element_size() >= nbytes and dst.numel() * dst.element_size() >= nbytes
    e0, e1 = ev.create(), ev.create()

    def timed(launch):
        ts = []
        for rep in range(4):
            ev.record(e0, stream)
            launch()
            ev.record(e1, stream)
            torch.cuda.synchronize()
            if rep > 0:
                ts.append(ev.ms(e0, e1))
        return sorted(ts)[1]

    out = {}
    for name, kind, moved in (("hbm_read_GBps", K.HQMQ_CEIL_READ, nbytes),
                              ("hbm_write_GBps", K.HQMQ_CEIL_WRITE, nbytes),
                              ("hbm_copy_GBps", K.HQMQ_CEIL_COPY, 2 * nbytes)):
        t = timed(lambda: K.hqmq_ceiling_stream(kind, src, dst, nbytes, stream))
        out[name] = moved / (t * 1e-3) / 1e9
    sink = torch.zeros(1, dtype=torch.float32, device=src.device)
    for name, kind, iters in (("valu_fma_f32_TFLOPs", K.HQMQ_CEIL_FMA_F32, 100000),
                              ("mfma_f32_16x16x4_TFLOPs", K.HQMQ_CEIL_MFMA_F32, 20000),
                              ("mfma_f16_32x32x8_TFLOPs", K.HQMQ_CEIL_MFMA_F16, 40000)):
        fl = []
        t = timed(lambda: fl.append(K.hqmq_ceiling_compute(kind, iters, sink, stream)))
        out[name] = fl[-1] / (t * 1e-3) / 1e12
    ev.destroy(e0)
    ev.destroy(e1)
    return out


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def kernel_hash() -> str:
    return source_hash(KERNEL_SRC)


def _counters(path: str, hash_key: str, src: str):
    """A committed counter summary, or None when it is missing or was taken
    from another kernel source."""
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get(hash_key) != source_hash(src):
        return None
    return t


def counters_for(kernel: str, path: str = None):
    """Counter summary of one kernel of the 128k workload (or of `path`)."""
    t = _counters(path or COUNTERS_FILE, "kernel_sha256_16", KERNEL_SRC)
    return None if t is None else t.get("kernels", {}).get(kernel)


def traffic_per_launch(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated, average over
    the K and V launches) from the committed counters, or None."""
    c = counters_for(kernel)
    if not c or "fetch_bytes" not in c or "write_bytes" not in c:
        return None
    return c["fetch_bytes"]["avg"] + c["write_bytes"]["avg"]


def attend_traffic_per_launch():
    """HBM bytes per attention launch (one layer of the decode-step workload)
    from the committed counters, or None when they were taken from another
    attention kernel source."""
    t = _counters(COUNTERS5_FILE, "attend_sha256_16", ATTEND_SRC)
    c = None if t is None else t.get("kernels", {}).get("attend_split_kernel")
    if not c or "fetch_bytes" not in c or "write_bytes" not in c:
        return None
    return c["fetch_bytes"]["avg"] + c["write_bytes"]["avg"]


def cpu_baseline(w, xs, cbs, seconds: float):
    """The oracle as it stands, timed on whole Med3x batches of the resident
    workload (copied to host first) until ``seconds`` of work are done."""
    import numpy as np
    import oracle as O
    B = w.med_batch_tokens or w.tokens
    rng = np.random.default_rng(12345)
    cpt = w.head_dim // 4
    staged = []
    n_stage = 48
    for i in range(n_stage):
        role = w.roles[i % len(w.roles)]
        l, h = int(rng.integers(w.layers)), int(rng.integers(w.heads))
        bi = int(rng.integers(max(1, w.tokens // B)))
        x = xs[role][l, h, bi * B:(bi + 1) * B].float().cpu().numpy()
        staged.append((x, cbs[role][l, h], bi * B))
    chunks, t0, i = 0, time.perf_counter(), 0
    while True:
        x, q, tok0 = staged[i % n_stage]
        r = O.encode_range(x, q, tok0, w.med_batch_tokens, w.med_C)
        O.decode_range(r["codes"], r["hnorm"], x.shape[0], w.head_dim, q,
                       r["side_pos"] if w.med_batch_tokens else None,
                       r["side_val"] if w.med_batch_tokens else None, tok0)
        chunks += x.shape[0] * cpt
        i += 1
        if time.perf_counter() - t0 >= seconds and i >= 2:
            break
    el = time.perf_counter() - t0
    return {"value": chunks / el, "unit": "chunks/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{i} Med3x batches of {B * cpt} chunks ({B} tokens) drawn from the "
                      f"{w.name} K/V tensors, oracle encode + decode each, {el:.1f} s"}


def copy_calibration():
    """A plain copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 31                               # 4 GiB of fp16
    a = torch.empty(n, dtype=torch.float16, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 2 * n, "launches": 3}))


def summarize_rocpd(db: str, match: str = "hqmq"):
    """Per-kernel table (calls, average / min / max duration) of a rocprofv3
    kernel-trace database, for the text summaries kept under profiles/."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), avg(duration), min(duration), max(duration), "
                     "sum(duration), max(grid_x), max(workgroup_x), max(vgpr_count), "
                     "max(accum_vgpr_count), max(lds_size) from kernels group by name "
                     "order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows)
    print("| kernel | calls | avg ms | min ms | max ms | % of GPU time | grid threads | block | "
          "arch VGPR | acc VGPR | LDS B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        if match and match not in r[0]:
            continue
        name = r[0].replace("(anonymous namespace)::", "").split("(")[0]
        print(f"| `{name}` | {r[1]} | {r[2] / 1e6:.4f} | {r[3] / 1e6:.4f} | {r[4] / 1e6:.4f} | "
              f"{100 * r[5] / total:.1f} | {r[6]} | {r[7]} | {r[8]} | {r[9]} | {r[10]} |")


def summarize_pmc(db: str):
    """Per-kernel average of each collected counter (per dispatch) of a
    rocprofv3 --pmc database, as JSON lines."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, counter_name, count(*), avg(value), min(value), max(value) "
                     "from counters_collection group by kernel_name, counter_name").fetchall()
    for r in rows:
        print(json.dumps({"kernel": r[0].replace("(anonymous namespace)::", "").split("(")[0],
                          "counter": r[1], "dispatches": r[2], "avg": r[3], "min": r[4], "max": r[5]}))


def _kernel_key(name: str) -> str:
    """'void hqmq::decode_kernel<false, true, false>' -> 'decode_kernel'."""
    n = name.split("(")[0].split("<")[0].replace("void ", "").strip()
    return n.split("::")[-1]


def summarize_counters(run_dir: str, workload: int):
    """Counter summary of one workload from the per-pass outputs of
    `bench.py --summarize-pmc` (files pA.jsonl: instruction counts, pB.jsonl:
    busy metrics, pC.jsonl / pD.jsonl: optional SQ cycle counters, pF.jsonl /
    pW.jsonl: FETCH_SIZE / WRITE_SIZE, pFc.jsonl / pWc.jsonl: the same two
    counters on --copy-calibration) in run_dir.
    Prints the JSON kept under profiles/: per kernel the counters' average,
    minimum and maximum over its dispatches (the minimum and maximum of the
    codec kernels are its V and K launches), instructions per chunk, and
    HBM bytes per dispatch scaled by the copy calibration."""
    import synth
    w = synth.WORKLOADS[workload]

    def load(tag):
        path = os.path.join(run_dir, f"{tag}.jsonl")
        out = {}
        if not os.path.exists(path):
            return out
        for line in open(path):
            r = json.loads(line)
            out.setdefault(r["kernel"], {})[r["counter"]] = r
        return out

    inst, busy, fetch, write = load("pA"), load("pB"), load("pF"), load("pW")
    cycles, more = load("pC"), load("pD")   # optional SQ cycle-counter passes
    cal_f = load("pFc").get("__amd_rocclr_copyBuffer", {}).get("FETCH_SIZE")
    cal_w = load("pWc").get("__amd_rocclr_copyBuffer", {}).get("WRITE_SIZE")
    moved_kib = 4 * 1024 * 1024          # the calibration copies 4 GiB each way
    fscale = moved_kib / cal_f["avg"] if cal_f else None
    wscale = moved_kib / cal_w["avg"] if cal_w else None
    chunks = w.layers * w.heads * w.tokens * w.head_dim // 4     # one role
    kernels = {}
    for name in sorted(set(inst) | set(busy)):
        if "hqmq" not in name:
            continue
        k = _kernel_key(name)
        e = kernels.setdefault(k, {"kernel": name})
        for src in (inst.get(name, {}), busy.get(name, {}), cycles.get(name, {}), more.get(name, {})):
            for c, r in src.items():
                e[c] = {"avg": r["avg"], "min": r["min"], "max": r["max"], "dispatches": r["dispatches"]}
        if name in fetch and fscale:
            e["fetch_bytes"] = {q: fetch[name]["FETCH_SIZE"][q] * 1024 * fscale for q in ("avg", "min", "max")}
        if name in write and wscale:
            e["write_bytes"] = {q: write[name]["WRITE_SIZE"][q] * 1024 * wscale for q in ("avg", "min", "max")}
        if k in ("encode_search_h_kernel", "encode_search_kernel", "decode_kernel") and "SQ_INSTS_VALU" in e:
            e["valu_insts_per_chunk"] = e["SQ_INSTS_VALU"]["avg"] / chunks
            e["valu_insts_per_wave_step_64_chunks"] = 64 * e["SQ_INSTS_VALU"]["avg"] / chunks
            e["mfma_insts_per_chunk"] = e["SQ_INSTS_MFMA"]["avg"] / chunks
            e["salu_insts_per_chunk"] = e["SQ_INSTS_SALU"]["avg"] / chunks
        if "SQ_ACTIVE_INST_VALU" in e and "SQ_ACTIVE_INST_VALU2" in e:
            # VALU issue: at most two instructions per quad-cycle per SIMD
            # (dual issue); quad-cycles with any = single + dual
            v, v2 = e["SQ_ACTIVE_INST_VALU"]["avg"], e["SQ_ACTIVE_INST_VALU2"]["avg"]
            e["valu_dual_issue_fraction"] = 2 * v2 / v if v else None
            e["valu_issue_quad_cycles"] = v - v2
        if "VALUBusy" in e:
            e["valu_busy"] = e["VALUBusy"]["avg"] / 100.0
            e["source"] = "VALUBusy = 100 sum(SQ_ACTIVE_INST_VALU) / CU_NUM / max(GRBM_GUI_ACTIVE) (rocprofv3's definition)"
    print(json.dumps({"workload": synth.describe(w), "chunks_per_role": chunks,
                      "fetch_scale": fscale, "write_scale": wscale,
                      "kernel_sha256_16": kernel_hash(),
                      "attend_sha256_16": source_hash(ATTEND_SRC),
                      "kernels": kernels}, indent=1))


def decode_step_bench(args, w, fakequant: bool = True):
    """Decode-step workload: the cache of ``w.sequences`` sequences (stacked on
    the token axis of every (layer, head)) is encoded once, untimed.  One step
    encodes the step's appended tokens (one per sequence, a Med3x batch of
    their own) for K and V and then runs the attention of every layer over the
    cache, read straight from the records (hqmq_attend, GQA group 4).  For
    comparison the same step is also timed the "fake-quant" way: decode the
    whole cache to fp16 (hqmq_decode, K and V) and run attention on it with
    torch's batched matmuls."""
    import math
    import torch
    import kv_cache_quantization_hqmq_amd as K
    import synth
    torch.cuda.set_device(0)
    sh = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    group = 4
    nf = NORM_FORMATS[args.norm_format]
    desc = K.Desc.make(w.layers, w.heads, w.tokens, w.head_dim, w.S, K.HQMQ_F16,
                       w.med_batch_tokens, w.med_C, nf)
    desc_a = K.Desc.make(w.layers, w.heads, w.append_tokens, w.head_dim, w.S, K.HQMQ_F16,
                         w.append_tokens, w.med_C, nf)
    sz, sza = K.hqmq_sizes(desc), K.hqmq_sizes(desc_a)
    L, H, D, nseq = w.layers, w.heads, w.head_dim, w.sequences
    Tc = w.tokens // nseq
    scale = 1.0 / math.sqrt(D)
    log(f"workload {synth.describe(w)}; {sz.chunks} cached + {sza.chunks} appended chunks per role")
    ys, cbs, recs, xa, reca, n_out = {}, {}, {}, {}, {}, {}
    ws = K.workspace(desc)
    ws_a = K.workspace(desc_a)
    for role in w.roles:
        t = time.perf_counter()
        ys[role] = synth.generate(w, role, "cuda")
        cbs[role] = torch.from_numpy(K.hqmq_make_codebook(w.codebook_seed, w.layers, w.heads,
                                                           role, w.S)).cuda()
        recs[role] = K.encode(desc, ys[role], cbs[role], ws=ws)
        n_out[role] = recs[role].n_outliers
        torch.cuda.synchronize()
        log(f"role {role}: cache generated and encoded in {time.perf_counter() - t:.1f} s, "
            f"{n_out[role]} outliers ({n_out[role] / sz.chunks:.4%})")
        xa[role] = [synth.generate_append(w, role, i, "cuda") for i in range(args.steps + args.warmup)]
        reca[role] = K.allocate_records(desc_a)
    del ws
    starts = torch.arange(nseq, dtype=torch.int64, device="cuda") * Tc
    lens = torch.full((nseq,), Tc, dtype=torch.int32, device="cuda")
    gq = torch.Generator(device="cuda")
    gq.manual_seed(4242)
    qs = torch.randn((L, nseq, H * group, D), generator=gq, device="cuda").to(torch.float16)
    adesc = [K.AttnDesc.make(nseq, group, l, Tc, scale) for l in range(L)]
    asz = K.hqmq_attn_sizes(desc, adesc[0])
    aws = torch.empty((int(asz.workspace_bytes),), dtype=torch.uint8, device="cuda")
    aout = torch.empty((L, nseq, H * group, D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def encode_appended(i):
        for role in w.roles:
            K.hqmq_encode(desc_a, xa[role][i], cbs[role], reca[role], ws_a, sh)

    def fused_step(i, e=None):
        if e:
            ev.record(e[0], sh)
        encode_appended(i)
        if e:
            ev.record(e[1], sh)
        for l in range(L):
            K.hqmq_attend(desc, adesc[l], recs[0], cbs[0], recs[1], cbs[1], qs[l], starts, lens,
                          aout[l], aws, sh)
        if e:
            ev.record(e[2], sh)

    def torch_attention(l):
        # decoded cache [H][nseq * Tc][D] -> [H * nseq, Tc, D]; contiguous operands only
        k = ys[0][l].view(H * nseq, Tc, D)
        v = ys[1][l].view(H * nseq, Tc, D)
        q = qs[l].view(nseq, H, group, D).transpose(0, 1).reshape(H * nseq, group, D)
        s = torch.bmm(k, q.transpose(1, 2).contiguous()).float() * scale
        p = torch.softmax(s, dim=1)
        return torch.bmm(p.transpose(1, 2).contiguous().to(torch.float16), v)

    def fakequant_step(i, e=None):
        if e:
            ev.record(e[0], sh)
        encode_appended(i)
        for role in w.roles:
            K.hqmq_decode(desc, recs[role], cbs[role], ys[role], sh)
        if e:
            ev.record(e[1], sh)
        for l in range(L):
            torch_attention(l)
        if e:
            ev.record(e[2], sh)

    def timed(fn, n_events):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        evs = [tuple(ev.create() for _ in range(n_events)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(args.warmup + i, evs[i])
        torch.cuda.synchronize()
        wall = 1000.0 * (time.perf_counter() - t0) / args.steps
        parts = [sum(ev.ms(e[j], e[j + 1]) for e in evs) / args.steps for j in range(n_events - 1)]
        for e in evs:
            for x in e:
                ev.destroy(x)
        return wall, parts

    log(f"timing {args.steps} fused steps")
    fused_ms, (enc_ms, att_ms) = timed(fused_step, 3)
    assert torch.isfinite(aout).all(), "attention produced non-finite values"
    if fakequant:
        log(f"timing {args.steps} fake-quant steps")
        fq_ms, (fq_dec_ms, fq_att_ms) = timed(fakequant_step, 3)
    else:
        fq_ms = fq_dec_ms = fq_att_ms = float("nan")
    app_out = {r: K.hqmq_encode_result(reca[r], sh) for r in w.roles}

    rec_bytes = sz.idx_bytes + sz.hnorm_bytes
    side = sum(12 * n_out[r] for r in w.roles)
    # one attention launch reads one layer's K and V records and side entries
    att_bytes = (2 * rec_bytes + side) / L + nseq * H * group * D * (2 + 4)
    att_launch_ms = att_ms / L
    att_gbps = att_bytes / (att_launch_ms * 1e-3) / 1e9
    dec_ms = fq_dec_ms - enc_ms
    dec_bytes = sum(rec_bytes + sz.chunks * 8 + 12 * n_out[r] + sz.offsets_bytes for r in w.roles)
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    roles = len(w.roles)
    work = roles * (sz.chunks + sza.chunks)
    out = {
        "metric": METRIC,
        "value": work / (fused_ms * 1e-3),
        "unit": "chunks/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": fused_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16xf16->f32 mfma attention, f32 decode",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "kv_heads": H, "query_heads": H * group,
                   "sequences": nseq, "cached_tokens_per_sequence": Tc,
                   "appended_tokens_per_step": w.append_tokens, "head_dim": D,
                   "roles": "K+V", "input": w.dtype, "S": w.S,
                   "med3_batch_tokens": w.med_batch_tokens, "med3_C": w.med_C,
                   "norm_format": args.norm_format,
                   "step": "encode appended tokens + attention of every layer read from the records",
                   "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": "attend (one layer)", "achieved": att_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": att_gbps / PEAK_HBM_GBPS,
                     # counters were taken on the binary16-norm configuration
                     "traffic": attend_traffic_per_launch() if args.norm_format == "f16" else None,
                     "algorithmic_per_launch": att_bytes, "avg_launch_ms": att_launch_ms},
        "encode_appended_ms": enc_ms,
        "attention_ms_per_step": att_ms,
        "fakequant": {"ms_per_step": fq_ms, "decode_ms": dec_ms, "torch_attention_ms": fq_att_ms,
                      "decode_roofline": {"bound": "hbm", "achieved": dec_gbps,
                                          "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                          "frac": dec_gbps / PEAK_HBM_GBPS,
                                          "algorithmic_per_launch": dec_bytes / roles,
                                          "avg_launch_ms": dec_ms / roles}},
        "fused_speedup_vs_fakequant": fq_ms / fused_ms,
        "appended_outliers_last_step": app_out,
        "cache_outlier_fraction": sum(n_out.values()) / (roles * sz.chunks),
        "cache_bits_per_element": 8 * sum(rec_bytes + 12 * n_out[r] + sz.offsets_bytes for r in w.roles)
        / (roles * sz.chunks * 4),
        "kernel_sha256_16": kernel_hash(),
        "cpu_baseline": None,
    }
    return out


def paged_step_bench(args, w):
    """Decode-step workload on paged pools, the serving form of the step: the
    cache of ``w.sequences`` sequences is appended into K and V pools of
    ``--page-tokens``-token pages (pages of a sequence scattered through the
    pool; prefill calls of one Med3x batch, 4096 tokens of one sequence,
    untimed).  One step appends the step's new token of every sequence
    (hqmq_append, K and V, Med3x batch = the step) and runs the attention of
    every layer over each sequence's pages including the new token
    (hqmq_attend_paged, GQA group 4)."""
    import math
    import numpy as np
    import torch
    import kv_cache_quantization_hqmq_amd as K
    import synth
    torch.cuda.set_device(0)
    sh = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    group = 4
    nf = NORM_FORMATS[args.norm_format]
    L, H, D, nseq = w.layers, w.heads, w.head_dim, w.sequences
    Tc = w.tokens // nseq
    cpt = D // 4
    P = args.page_tokens
    total = args.warmup + args.steps
    pps = (Tc + total + P - 1) // P            # pages per sequence
    NP = nseq * pps
    cap = P * cpt // 16                         # side entries per page: 6.25% of its chunks
    pdesc = K.PagedDesc(NP, P, cap)
    B = w.med_batch_tokens
    desc0 = K.Desc.make(L, H, 0, D, w.S, K.HQMQ_F16, B, w.med_C, nf)
    desc_p = K.Desc.make(L, H, B, D, w.S, K.HQMQ_F16, B, w.med_C, nf)           # prefill call
    desc_a = K.Desc.make(L, H, nseq, D, w.S, K.HQMQ_F16, nseq, w.med_C, nf)     # one step
    rng = np.random.default_rng(7)
    ptab = rng.permutation(NP).astype(np.int32).reshape(nseq, pps)
    ptab_d = torch.from_numpy(ptab).cuda()
    psz = K.hqmq_paged_sizes(desc0, pdesc)
    pool_bytes = psz.idx_bytes + psz.hnorm_bytes + psz.side_count_bytes + psz.side_pos_bytes + psz.side_val_bytes
    log(f"workload {synth.describe(w)}; paged pools: {NP} pages of {P} tokens, {cap} side entries per page, "
        f"{pool_bytes / 1e9:.1f} GB per role")
    pools, cbs, xa = {}, {}, {}
    ws_p = K.append_workspace(desc_p, pdesc)
    n_pre = {}
    for role in w.roles:
        t = time.perf_counter()
        cbs[role] = torch.from_numpy(K.hqmq_make_codebook(w.codebook_seed, L, H, role, w.S)).cuda()
        pools[role] = K.allocate_pool(desc0, pdesc)
        x_all = synth.generate(w, role, "cuda")
        st = torch.zeros(2, dtype=torch.int64, device="cuda")
        st_sum = torch.zeros(2, dtype=torch.int64, device="cuda")
        tok = torch.arange(B, dtype=torch.int64, device="cuda")
        for q in range(nseq):
            for k0 in range(0, Tc, B):
                x = x_all[:, :, q * Tc + k0:q * Tc + k0 + B].contiguous()
                t_seq = k0 + tok
                slots = ptab_d[q].long()[t_seq // P] * P + t_seq % P
                K.hqmq_append(desc_p, pdesc, x, slots, cbs[role], pools[role], st, ws_p, sh)
                st_sum += st
        del x_all, x
        torch.cuda.synchronize()
        n_pre[role] = st_sum.cpu().tolist()
        log(f"role {role}: cache appended in {time.perf_counter() - t:.1f} s, {n_pre[role][0]} outliers, "
            f"{n_pre[role][1]} dropped (page lists full)")
        xa[role] = [synth.generate_append(w, role, i, "cuda") for i in range(total)]
    del ws_p
    ws_a = K.append_workspace(desc_a, pdesc)
    seqs = torch.arange(nseq, dtype=torch.int64, device="cuda")
    slots_i, lens_i = [], []
    for i in range(total):
        t = Tc + i
        slots_i.append((ptab_d[:, t // P].long() * P + t % P).contiguous())
        lens_i.append(torch.full((nseq,), t + 1, dtype=torch.int32, device="cuda"))
    gq = torch.Generator(device="cuda")
    gq.manual_seed(4242)
    qs = torch.randn((L, nseq, H * group, D), generator=gq, device="cuda").to(torch.float16)
    scale = 1.0 / math.sqrt(D)
    max_len = Tc + total
    adesc = [K.AttnDesc.make(nseq, group, l, max_len, scale) for l in range(L)]
    asz = K.hqmq_attn_sizes(desc0, adesc[0])
    aws = torch.empty((int(asz.workspace_bytes),), dtype=torch.uint8, device="cuda")
    aout = torch.empty((L, nseq, H * group, D), dtype=torch.float32, device="cuda")
    st_a = {r: torch.zeros(2, dtype=torch.int64, device="cuda") for r in w.roles}
    torch.cuda.synchronize()

    def step(i, e=None):
        if e:
            ev.record(e[0], sh)
        for role in w.roles:
            K.hqmq_append(desc_a, pdesc, xa[role][i], slots_i[i], cbs[role], pools[role], st_a[role], ws_a, sh)
        if e:
            ev.record(e[1], sh)
        for l in range(L):
            K.hqmq_attend_paged(desc0, pdesc, adesc[l], pools[0], cbs[0], pools[1], cbs[1], qs[l], ptab_d,
                                lens_i[i], aout[l], aws, sh)
        if e:
            ev.record(e[2], sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [tuple(ev.create() for _ in range(3)) for _ in range(args.steps)]
    log(f"timing {args.steps} paged steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    ms = 1000.0 * (time.perf_counter() - t0) / args.steps
    app_ms = sum(ev.ms(e[0], e[1]) for e in evs) / args.steps
    att_ms = sum(ev.ms(e[1], e[2]) for e in evs) / args.steps
    for e in evs:
        for x in e:
            ev.destroy(x)
    assert torch.isfinite(aout).all(), "attention produced non-finite values"
    app_out = {r: st_a[r].cpu().tolist() for r in w.roles}

    # one attention launch reads one layer's K and V records of every token and their side entries
    W = K.hqmq_sizes(desc0).words_per_token
    tok_all = nseq * (Tc + args.warmup + (args.steps + 1) / 2)   # mean over the timed steps
    rec_tok = W * 4 + (W * 4 if nf else cpt * 2)
    side = sum(n_pre[r][0] - n_pre[r][1] for r in w.roles) * 12 / L
    att_bytes = 2 * H * tok_all * rec_tok + side + nseq * H * group * D * (2 + 4)
    att_launch_ms = att_ms / L
    att_gbps = att_bytes / (att_launch_ms * 1e-3) / 1e9
    roles = len(w.roles)
    work = roles * H * L * tok_all * cpt
    out = {
        "metric": METRIC,
        "value": work / (ms * 1e-3),
        "unit": "chunks/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16xf16->f32 mfma attention, f32 decode",
        "data": "synthetic",
        "config": {"workload": w.name + "-paged", "layers": L, "kv_heads": H, "query_heads": H * group,
                   "sequences": nseq, "cached_tokens_per_sequence": Tc, "head_dim": D, "roles": "K+V",
                   "S": w.S, "med3_batch_tokens": B, "med3_C": w.med_C, "norm_format": args.norm_format,
                   "page_tokens": P, "pages": NP, "page_capacity": cap,
                   "step": "append the step's token of every sequence into the pools + attention of every "
                           "layer over each sequence's pages", "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": "attend_paged (one layer)", "achieved": att_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": att_gbps / PEAK_HBM_GBPS,
                     "traffic": None, "algorithmic_per_launch": att_bytes, "avg_launch_ms": att_launch_ms},
        "append_ms": app_ms,
        "attention_ms_per_step": att_ms,
        "prefill_outliers_dropped": {r: n_pre[r] for r in w.roles},
        "appended_outliers_last_step": app_out,
        "pool_bytes_per_role": pool_bytes,
        "kernel_sha256_16": kernel_hash(),
        "cpu_baseline": None,
    }
    return out


def _int_per_token(x, bits: int):
    """Naive symmetric per-(token, head) integer quantisation of x [..., D]
    (absmax scale in fp16, round to nearest): the baseline the pages compare
    against, as a torch reference for the quality report."""
    import torch
    qmax = 2 ** (bits - 1) - 1
    xf = x.float()
    scale = (xf.abs().amax(dim=-1, keepdim=True) / qmax).to(torch.float16).float()
    q = torch.where(scale > 0, torch.round(xf / scale.clamp_min(1e-30)), torch.zeros_like(xf)).clamp(-qmax, qmax)
    return (q * scale).to(x.dtype)


def _errors(x, y, q=None, scale=None):
    """Relative MSE, mean cosine of 4-element chunks' directions (degrees of
    the mean angle), mean cosine of head vectors, and, for queries q, the
    relative error of single-query attention outputs over the tokens of
    every (layer, head) (fp32 softmax of q k / sqrt(D), values y vs x)."""
    import torch
    xf, yf = x.float(), y.float()
    rel = float(((yf - xf) ** 2).sum() / (xf ** 2).sum())
    xc, yc = xf.reshape(-1, 4), yf.reshape(-1, 4)
    nx, ny = xc.norm(dim=1), yc.norm(dim=1)
    ok = (nx > 0) & (ny > 0)
    cosc = ((xc * yc).sum(dim=1)[ok] / (nx[ok] * ny[ok])).clamp(-1, 1)
    ang = float(torch.rad2deg(torch.acos(cosc)).mean())
    cosv = float(torch.nn.functional.cosine_similarity(xf.reshape(-1, xf.shape[-1]),
                                                       yf.reshape(-1, yf.shape[-1]), dim=1).mean())
    out = {"rel_mse": rel, "chunk_angle_deg": ang, "vector_cosine": cosv}
    return out


def _attention_error(kx, vx, ky, vy, q, scale):
    """Relative error of single-query attention outputs with (ky, vy) in
    place of (kx, vx): kx.. [L, H, T, D], q [L, H, D]; fp32 throughout."""
    import torch
    L, H, T, D = kx.shape
    num, den = 0.0, 0.0
    for l in range(L):
        qf = q[l].float().unsqueeze(1)                      # [H, 1, D]
        ref = torch.softmax(torch.bmm(qf, kx[l].float().transpose(1, 2).contiguous()) * scale, -1)
        ref = torch.bmm(ref, vx[l].float())
        got = torch.softmax(torch.bmm(qf, ky[l].float().transpose(1, 2).contiguous()) * scale, -1)
        got = torch.bmm(got, vy[l].float())
        num += float(((got - ref) ** 2).sum())
        den += float((ref ** 2).sum())
    return (num / den) ** 0.5


def quality_report(args):
    """Reconstruction quality on the synthetic inputs (no model weights or
    datasets exist here): the covering trend of the random multiplicative
    codebook against S (Prop. 3.1 gives only O((24 S)^(-1/3))), Med3x on
    outlier-heavy inputs, and naive per-token integer quantisation at several
    widths, each with its storage cost in bits per element."""
    import math
    import numpy as np
    import torch
    import kv_cache_quantization_hqmq_amd as K
    import synth
    torch.cuda.set_device(0)
    rep = {"report": "HQMQ reconstruction quality on synthetic KV tensors (one MI355X)", "data": "synthetic"}

    def run(w, x, role, S, B, nf=0):
        desc = K.Desc.make(w.layers, w.heads, w.tokens, w.head_dim, S, K.HQMQ_F16, B, 3.0, nf)
        cb = torch.from_numpy(K.hqmq_make_codebook(w.codebook_seed, w.layers, w.heads, role, S)).cuda()
        rec = K.encode(desc, x, cb)
        y = K.decode(desc, rec, cb)
        sz = K.hqmq_sizes(desc)
        nbytes = sz.idx_bytes + sz.hnorm_bytes + 12 * rec.n_outliers + sz.offsets_bytes + sz.codebook_bytes
        return y, 8.0 * nbytes / (sz.chunks * 4), rec.n_outliers / sz.chunks

    # 1) covering trend on i.i.d. N(0,1) (every direction equally likely)
    w = synth.WORKLOADS[2].scaled(layers=4, heads=8, tokens=8192, dist="normal", data_seed=4401)
    x = synth.generate(w, 0, "cuda")
    trend = []
    for S in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        y, bits, _ = run(w, x, 0, S, 0)
        e = _errors(x, y)
        trend.append({"S": S, "codewords": 24 * S, "bits_per_element": bits, **e})
        log(f"S={S}: {e}")
        del y
    xs = np.log([t["codewords"] for t in trend])
    slope = float(np.polyfit(xs, np.log([t["chunk_angle_deg"] for t in trend]), 1)[0])
    rep["covering_trend"] = {"workload": f"N(0,1) [{w.layers}, {w.heads}, {w.tokens}, {w.head_dim}] fp16",
                             "points": trend, "angle_vs_codewords_loglog_slope": slope,
                             "expected_slope": -1.0 / 3.0}
    del x

    # 2) outlier-heavy and lognormal-channel K/V: HQMQ (Med3x on/off) vs int-k per token
    cases = [(synth.WORKLOADS[3].scaled(layers=4, heads=4, tokens=8192, data_seed=4402), 32),
             (synth.WORKLOADS[2].scaled(layers=4, heads=8, tokens=8192, data_seed=4403), 8)]
    rep["comparisons"] = []
    for w, S in cases:
        xs_ = {r: synth.generate(w, r, "cuda") for r in (0, 1)}
        g = torch.Generator(device="cuda")
        g.manual_seed(77)
        q = torch.randn((w.layers, w.heads, w.head_dim), generator=g, device="cuda").to(torch.float16)
        sc = 1.0 / math.sqrt(w.head_dim)
        rows = []
        variants = [("hqmq_med3", S, 4096, 0), ("hqmq_no_med3", S, 0, 0),
                    ("hqmq_med3_packed_norms", S, 4096, 1), ("hqmq_no_med3_packed_norms", S, 0, 1)]
        for name, SS, B, nf in variants:
            ys, bits, fo = {}, 0.0, 0.0
            for r in (0, 1):
                ys[r], b_, f_ = run(w, xs_[r], r, SS, B, nf)
                bits += b_ / 2
                fo += f_ / 2
            e = _errors(torch.cat([xs_[0], xs_[1]]), torch.cat([ys[0], ys[1]]))
            e["attention_rel_error"] = _attention_error(xs_[0], xs_[1], ys[0], ys[1], q, sc)
            rows.append({"method": name, "S": SS, "med3_batch_tokens": B, "bits_per_element": bits,
                         "outlier_fraction": fo, **e})
            log(f"{w.name} {name}: {rows[-1]}")
        for bw in (4, 6, 8):
            ys = {r: _int_per_token(xs_[r], bw) for r in (0, 1)}
            e = _errors(torch.cat([xs_[0], xs_[1]]), torch.cat([ys[0], ys[1]]))
            e["attention_rel_error"] = _attention_error(xs_[0], xs_[1], ys[0], ys[1], q, sc)
            rows.append({"method": f"int{bw}_per_token", "bits_per_element": bw + 16.0 / w.head_dim, **e})
            log(f"{w.name} int{bw}: {rows[-1]}")
        rep["comparisons"].append({"workload": synth.describe(w), "rows": rows})
    print(json.dumps(rep), flush=True)


def codec_bench(w, norm_format: str, xs, cbs, ev, sh, steps: int, warmup: int, ws=None, ys=None,
                overlap: int = 0) -> dict:
    """Time `steps` steps of the codec on workload w's resident inputs xs
    (dict role -> device tensor) in one norm format: per role hqmq_encode
    (search kernel bracketed by HIP events the library records on the launch
    stream) and hqmq_decode.  overlap = 0: every call on one stream, the
    encodes then the decodes.  overlap = n > 0: each role's decode runs on a
    second stream as soon as its encode is done, beside the next encode, with
    the search capped at n blocks per CU (hqmq_set_search_blocks_per_cu) so
    that the decode finds room; a role's encode waits for the previous decode
    of its records.  Returns the figures and keeps the records and decode
    outputs in the result ('_recs', '_ys')."""
    import torch
    import kv_cache_quantization_hqmq_amd as K
    desc = K.Desc.make(w.layers, w.heads, w.tokens, w.head_dim, w.S,
                       K.HQMQ_F32 if w.dtype == "f32" else K.HQMQ_F16, w.med_batch_tokens, w.med_C,
                       NORM_FORMATS[norm_format])
    sz = K.hqmq_sizes(desc)
    if ws is None or (sz.workspace_bytes and ws.numel() < sz.workspace_bytes):
        ws = K.workspace(desc, "cuda")
    recs = {}
    ys = {} if ys is None else ys
    for role in w.roles:
        # size the side list from a first encode (re-allocated on overflow)
        recs[role] = K.encode(desc, xs[role], cbs[role], ws=ws)
        if recs[role].capacity > 0 and recs[role].n_outliers > 0:
            cap = int(recs[role].n_outliers)
            if cap < recs[role].capacity // 2:
                recs[role] = K.encode(desc, xs[role], cbs[role], capacity=cap, ws=ws)
        if role not in ys:
            ys[role] = torch.empty(desc.shape, dtype=w.torch_dtype, device="cuda")
        log(f"{norm_format} norms, role {role}: {recs[role].n_outliers} outliers "
            f"({recs[role].n_outliers / sz.chunks:.4%})")
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream() if overlap else None   # default priority
    enc_done = {r: torch.cuda.Event() for r in w.roles}
    dec_done = {r: torch.cuda.Event() for r in w.roles}
    K.hqmq_set_search_blocks_per_cu(overlap)

    def encode(role, events):
        e = events[("enc", role)] if events else None
        if e:
            ev.record(e[0], sh)
        K.hqmq_encode_timed(desc, xs[role], cbs[role], recs[role], ws, sh,
                            e[1] if e else None, e[2] if e else None)
        if e:
            ev.record(e[3], sh)

    def decode(role, events, stream):
        d = events[("dec", role)] if events else None
        if d:
            ev.record(d[0], stream)
        K.hqmq_decode(desc, recs[role], cbs[role], ys[role], stream)
        if d:
            ev.record(d[1], stream)

    def step(events=None):
        if not overlap:
            for role in w.roles:
                encode(role, events)
            for role in w.roles:
                decode(role, events, sh)
            return
        for role in w.roles:
            main.wait_event(dec_done[role])     # the last decode of these records
            encode(role, events)
            enc_done[role].record(main)
            side.wait_event(enc_done[role])
            decode(role, events, side.cuda_stream)
            dec_done[role].record(side)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    all_events = [{**{("enc", r): tuple(ev.create() for _ in range(4)) for r in w.roles},
                   **{("dec", r): tuple(ev.create() for _ in range(2)) for r in w.roles}}
                  for _ in range(steps)]
    log(f"timing {steps} steps ({norm_format} norms)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(all_events[i])
    torch.cuda.synchronize()
    ms_step = 1000.0 * (time.perf_counter() - t0) / steps
    K.hqmq_set_search_blocks_per_cu(0)

    search_ms = {r: [] for r in w.roles}
    enc_ms = {r: [] for r in w.roles}
    dec_ms = {r: [] for r in w.roles}
    for evs in all_events:
        for r in w.roles:
            a, b, c, d = evs[("enc", r)]
            search_ms[r].append(ev.ms(b, c))
            enc_ms[r].append(ev.ms(a, d))
            e0, e1 = evs[("dec", r)]
            dec_ms[r].append(ev.ms(e0, e1))
        for v in evs.values():
            for e in v:
                ev.destroy(e)
    mean = lambda v: sum(v) / len(v)
    flat = lambda d: [x for r in w.roles for x in d[r]]
    dec_in_step = dec_ms
    if overlap:
        # in the overlapped step a decode shares the chip with an encode; its
        # kernel figures come from each role's decode run alone
        dec_ms = {r: [] for r in w.roles}
        for r in w.roles:
            pairs = [(ev.create(), ev.create()) for _ in range(3)]
            for a_, b_ in pairs:
                ev.record(a_, sh)
                K.hqmq_decode(desc, recs[r], cbs[r], ys[r], sh)
                ev.record(b_, sh)
            torch.cuda.synchronize()
            dec_ms[r] = [ev.ms(a_, b_) for a_, b_ in pairs]
            for a_, b_ in pairs:
                ev.destroy(a_)
                ev.destroy(b_)

    # every launch must still be valid after the timed steps
    n_out = {r: K.hqmq_encode_result(recs[r], sh) for r in w.roles}
    chunks_role = sz.chunks
    total_chunks = chunks_role * len(w.roles)
    rec_bytes = sz.idx_bytes + (0 if norm_format == "exact" else sz.hnorm_bytes)
    comp_bytes = sum(rec_bytes + 12 * n_out[r] + sz.offsets_bytes + sz.codebook_bytes for r in w.roles)
    dec_bytes = {r: rec_bytes + chunks_role * (16 if w.dtype == "f32" else 8) + 12 * n_out[r] + sz.offsets_bytes
                 for r in w.roles}
    res = {
        "ms_per_step": ms_step,
        "search_ms": mean(flat(search_ms)),
        "search_ms_per_role": {str(r): mean(search_ms[r]) for r in w.roles},
        "encode_ms_per_role": {str(r): mean(enc_ms[r]) for r in w.roles},
        "med3_ms_per_role": {str(r): mean(enc_ms[r]) - mean(search_ms[r]) for r in w.roles},
        "decode_ms_per_role": {str(r): mean(dec_ms[r]) for r in w.roles},
        **({"decode_in_step_ms_per_role": {str(r): mean(dec_in_step[r]) for r in w.roles},
            "overlap_search_blocks_per_cu": overlap} if overlap else {}),
        "decode_GBps_per_role": {str(r): dec_bytes[r] / (mean(dec_ms[r]) * 1e-3) / 1e9 for r in w.roles},
        "decode_bytes_per_launch": mean([dec_bytes[r] for r in w.roles]),
        "decode_ms": mean(flat(dec_ms)),
        "encode_chunks_per_s": total_chunks / (sum(flat(enc_ms)) / steps * 1e-3),
        "decode_chunks_per_s": total_chunks / (sum(flat(dec_ms)) / steps * 1e-3),
        "encode_GBps_fp16_in": total_chunks * 8 / (sum(flat(enc_ms)) / steps * 1e-3) / 1e9,
        "decode_GBps_fp16_out": total_chunks * 8 / (sum(flat(dec_ms)) / steps * 1e-3) / 1e9,
        "value": total_chunks / (ms_step * 1e-3),
        "outlier_fraction": sum(n_out.values()) / total_chunks,
        "outliers_per_role": {str(r): n_out[r] for r in w.roles},
        "fp16_bytes": total_chunks * 8,
        "compressed_bytes": comp_bytes,
        "compression_ratio": total_chunks * 8 / comp_bytes,
        "bits_per_element": 8 * comp_bytes / (total_chunks * 4),
        "bulk_bits_per_element": 8 * rec_bytes / (chunks_role * 4),
        "_recs": recs, "_ys": ys, "_ws": ws, "_sz": sz,
    }
    return res


def public(d: dict) -> dict:
    return {k: v for k, v in d.items() if not k.startswith("_")}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--overlap", type=int, default=0, metavar="N",
                    help="encode/decode workloads: run each role's decode on a second stream beside the next "
                         "encode, the search capped at N blocks per CU (1..7; 0: one stream)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, help="1..5 (see synth.WORKLOADS; 5 is the decode step)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--paged", action="store_true",
                    help="workload 5 on paged pools (append + paged attention per step)")
    ap.add_argument("--page-tokens", type=int, default=128)
    ap.add_argument("--norm-format", choices=sorted(NORM_FORMATS), default="f16",
                    help="norm records: binary16 half-norms, packed b-bit compact codes, or exact-rate groups")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the main line: skip the other norm formats and the decode-step figures")
    ap.add_argument("--extra-steps", type=int, default=3, help="timed steps of each extra figure")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--quality", action="store_true", help="print the synthetic quality report instead")
    ap.add_argument("--summarize", metavar="ROCPD_DB", help="print a kernel table of a rocprofv3 database")
    ap.add_argument("--summarize-pmc", metavar="ROCPD_DB", help="print per-kernel counter averages")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="JSON counter summary of --workload from the --summarize-pmc outputs in DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize_rocpd(args.summarize)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the codec shards by (layer, head) with no "
              f"exchange, so there is no multi-GPU path to time (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_quantization_hqmq_amd as K
    import synth

    if args.copy_calibration:
        copy_calibration()
        return
    if args.quality:
        quality_report(args)
        return

    w = synth.WORKLOADS[args.workload]
    if w.sequences > 1:
        if args.paged:
            out = paged_step_bench(args, w)
        else:
            out = decode_step_bench(args, w)
        print(json.dumps(out), flush=True)
        return
    dev = "cuda"
    torch.cuda.set_device(0)
    sh = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    log(f"workload {synth.describe(w)}")

    xs, cbs_host, cbs = {}, {}, {}
    for role in w.roles:
        t = time.perf_counter()
        xs[role] = synth.generate(w, role, dev)
        cbs_host[role] = K.hqmq_make_codebook(w.codebook_seed, w.layers, w.heads, role, w.S)
        cbs[role] = torch.from_numpy(cbs_host[role]).to(dev)
        torch.cuda.synchronize()
        log(f"role {role}: input generated in {time.perf_counter() - t:.1f} s")

    main_res = codec_bench(w, args.norm_format, xs, cbs, ev, sh, args.steps, args.warmup, overlap=args.overlap)
    sz = main_res["_sz"]
    chunks_role = sz.chunks
    total_chunks = chunks_role * len(w.roles)

    # encode search: the method's arithmetic is 16 S FMA per chunk; it runs on
    # the f16 matrix cores (v_mfma_f32_32x32x8_f16 with the codebook split into
    # two binary16 parts, so the instructions issue twice those flops); the
    # contraction's roofline is that instruction's dense f16 peak, and the
    # counters show the VALU epilogue is what binds
    flops_launch = 32 * w.S * chunks_role
    s_ms = main_res["search_ms"]
    achieved_tf = flops_launch / (s_ms * 1e-3) / 1e12
    search_bytes = chunks_role * (16 if w.dtype == "f32" else 8) + sz.idx_bytes + sz.hnorm_bytes
    # counters were taken on the binary16-norm configuration
    is_ref_cfg = w.wid == 4 and args.norm_format == "f16"
    traffic = traffic_per_launch("encode_search_h_kernel") if is_ref_cfg else None
    cnt = counters_for("encode_search_h_kernel") if is_ref_cfg else None
    d_ms = main_res["decode_ms"]
    dec_bytes_launch = main_res["decode_bytes_per_launch"]
    dec_gbps = dec_bytes_launch / (d_ms * 1e-3) / 1e9
    roofline = {"bound": "mfma", "kernel": "encode_search", "instruction": "v_mfma_f32_32x32x8_f16",
                "achieved": achieved_tf, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved_tf / PEAK_F16_MFMA_TFLOPS, "traffic": traffic,
                "algorithmic_per_launch": flops_launch, "avg_launch_ms": s_ms,
                "issued_mfma_flops_per_launch": 2 * 16384 * ((w.S + 7) // 8) * (chunks_role // 64)
                if w.dtype == "f16" else None,
                "hbm_bytes_per_launch": search_bytes,
                "hbm_frac": search_bytes / (s_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "frac_of_fp32_peak": achieved_tf / PEAK_FP32_TFLOPS}
    if cnt:
        roofline["valu"] = {k: cnt[k] for k in ("valu_insts_per_wave_step_64_chunks", "mfma_insts_per_chunk",
                                                 "valu_busy", "source") if k in cnt}
        if "MfmaUtil" in cnt:
            roofline["valu"]["mfma_util"] = cnt["MfmaUtil"]["avg"] / 100.0
    out = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "chunks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 mfma search, f32 decode" if w.dtype == "f16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "kv_heads": w.heads,
                   "tokens": w.tokens, "head_dim": w.head_dim, "roles": "K+V" if len(w.roles) == 2 else "K",
                   "input": w.dtype, "S": w.S, "med3_batch_tokens": w.med_batch_tokens,
                   "med3_C": w.med_C, "norm_format": args.norm_format, "parallelism": "none"},
        "roofline": roofline,
        "roofline_decode": {"bound": "hbm", "kernel": "decode", "achieved": dec_gbps,
                            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": dec_gbps / PEAK_HBM_GBPS,
                            "traffic": traffic_per_launch("decode_kernel") if is_ref_cfg else None,
                            "algorithmic_per_launch": dec_bytes_launch, "avg_launch_ms": d_ms,
                            "avg_launch_ms_per_role": main_res["decode_ms_per_role"],
                            "GBps_per_role": main_res["decode_GBps_per_role"]},
        **{k: v for k, v in public(main_res).items()
           if k not in ("ms_per_step", "value", "decode_ms", "decode_bytes_per_launch")},
        "kernel_sha256_16": kernel_hash(),
    }
    if not args.no_ceilings and len(w.roles) == 2 and main_res["_ys"][w.roles[0]].numel() * 2 >= (4 << 30):
        # measured ceilings (context; the decode outputs serve as scratch)
        ys = main_res["_ys"]
        c = measure_ceilings(ys[w.roles[0]], ys[w.roles[1]], sh, ev)
        dec_read = dec_bytes_launch - chunks_role * 8
        dec_write = chunks_role * 8
        mix = (dec_read + dec_write) / (dec_read / c["hbm_read_GBps"] + dec_write / c["hbm_write_GBps"])
        out["ceilings"] = dict(c, decode_mix_GBps=mix)
        out["roofline"]["frac_of_measured_mfma_f16"] = achieved_tf / c["mfma_f16_32x32x8_TFLOPs"]
        out["roofline_decode"]["frac_of_measured_mix"] = dec_gbps / mix
        out["roofline_decode"]["frac_of_measured_copy"] = dec_gbps / c["hbm_copy_GBps"]
    if not args.no_cpu_baseline:
        log("timing the oracle on a host sample")
        out["cpu_baseline"] = cpu_baseline(w, xs, cbs_host, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None

    if not args.no_extras and w.wid == 4:
        # the same step with the other norm formats, on the same inputs
        ws, ys = main_res["_ws"], main_res["_ys"]
        del main_res
        out["formats"] = {}
        for fmt in sorted(NORM_FORMATS):
            if fmt == args.norm_format:
                continue
            torch.cuda.empty_cache()
            r = codec_bench(w, fmt, xs, cbs, ev, sh, args.extra_steps, 1, ws=None, ys=ys, overlap=args.overlap)
            keep = ("ms_per_step", "search_ms", "med3_ms_per_role", "decode_ms_per_role", "decode_GBps_per_role",
                    "compression_ratio", "bits_per_element", "bulk_bits_per_element", "compressed_bytes")
            out["formats"][fmt] = {k: r[k] for k in keep}
            out["formats"][fmt]["decode_frac_of_hbm_peak"] = \
                r["decode_bytes_per_launch"] / (r["decode_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS
            out["formats"][fmt]["steps"] = args.extra_steps
            del r
        del xs, ys, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        # the decode-step workload (attention read from the records)
        a5 = argparse.Namespace(**vars(args))
        a5.steps, a5.warmup, a5.norm_format = args.extra_steps, 1, "f16"
        d = decode_step_bench(a5, synth.WORKLOADS[5])
        out["decode_step"] = {k: d[k] for k in ("ms_per_step", "value", "unit", "config", "roofline",
                                                "encode_appended_ms", "attention_ms_per_step", "fakequant",
                                                "fused_speedup_vs_fakequant", "cache_bits_per_element")}
        out["decode_step"]["steps"] = a5.steps
        del d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        a5.norm_format = "exact"
        d = decode_step_bench(a5, synth.WORKLOADS[5], fakequant=False)
        out["decode_step"]["exact_records"] = {k: d[k] for k in ("ms_per_step", "roofline", "attention_ms_per_step",
                                                                 "cache_bits_per_element")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
