"""Paged pools through the C ABI compared with a model of the pool built
from the oracle.

A scenario is a sequence of append calls.  Each call appends consecutive
tokens of some sequences (prefill: many, decode: one per sequence) to the
pages those sequences own; pages come from a shuffled free list, so a
sequence's pages are scattered through the pool.  The model replays the
calls with the oracle: every call's tokens are encoded as one tensor
(``encode_range`` with the call's Med3x batches), each token's codes and
half-norm go to its slot, and each page's side list takes the call's outlier
entries of that page in order, up to the page capacity (entries past it are
dropped and their chunks keep the bulk record, flag cleared).

Records must match the model bit for bit, except index codes where the
oracle's top-2 gap is below 1e-6 (both choices are correct there; the
model then takes the GPU's code for the decoded values).  Attention over the
pages is compared with the oracle's plain attention over the model's decoded
values with the bound derived in tests/attend_cases.py.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import kv_cache_quantization_hqmq_amd as K
import oracle as O
from tests import attend_cases as A
from tests import parity as P


@dataclass
class Scenario:
    layers: int = 2
    heads: int = 2
    head_dim: int = 128
    S: int = 32
    med_batch_tokens: int = 1 << 20   # the whole call is one Med3x batch per (layer, head)
    med_C: float = 3.0
    norm_format: int = K.HQMQ_NORM_F16
    num_pages: int = 24
    page_tokens: int = 64
    page_capacity: int = 256
    # calls: lists of (sequence, tokens appended)
    calls: list = field(default_factory=lambda: [
        [(0, 200), (1, 64), (2, 1), (4, 130)],
        [(0, 1), (1, 1), (2, 1), (3, 1), (4, 1)],
        [(3, 70), (5, 5)],
        [(0, 1), (2, 1), (3, 1), (4, 1), (5, 1)],
    ])
    seed: int = 0
    outlier_channels: int = 1


def _desc(sc: Scenario, tokens: int) -> K.Desc:
    return K.Desc.make(sc.layers, sc.heads, tokens, sc.head_dim, sc.S, K.HQMQ_F16, sc.med_batch_tokens,
                       sc.med_C, sc.norm_format)


def _pdesc(sc: Scenario) -> K.PagedDesc:
    return K.PagedDesc(sc.num_pages, sc.page_tokens, sc.page_capacity)


def _call_input(sc: Scenario, i: int, T: int) -> torch.Tensor:
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * sc.seed + i)
    x = torch.randn((sc.layers, sc.heads, T, sc.head_dim), generator=g, device="cuda")
    # hot channels (Med3x outliers) and a few token spikes
    for c in range(sc.outlier_channels):
        x[:, :, :, 7 + 19 * c] *= 30.0
    x[:, :, ::37, :] *= 6.0
    return x.to(torch.float16)


class PoolModel:
    """The pool a sequence of appends should leave, from the oracle."""

    def __init__(self, sc: Scenario, cb_host: np.ndarray):
        self.sc, self.cb = sc, cb_host
        L, H, NP, P_ = sc.layers, sc.heads, sc.num_pages, sc.page_tokens
        self.cpt = sc.head_dim // 4
        self.codes = np.zeros((L, H, NP, P_, self.cpt), np.int64)
        self.gap = np.full((L, H, NP, P_, self.cpt), np.inf)
        self.h16 = np.zeros((L, H, NP, P_, self.cpt), np.uint16)
        self.side = [[[[] for _ in range(NP)] for _ in range(H)] for _ in range(L)]
        self.written = np.zeros((NP, P_), bool)
        self.found = []     # per call: outliers
        self.dropped = []   # per call: entries dropped (page list full)

    def apply(self, x: np.ndarray, slots: np.ndarray):
        sc, cpt = self.sc, self.cpt
        T = x.shape[2]
        B = sc.med_batch_tokens
        found = dropped = 0
        for l in range(sc.layers):
            for h in range(sc.heads):
                r = O.encode_range(x[l, h], self.cb[l, h], 0, B, sc.med_C)
                codes = r["codes"].reshape(T, cpt)
                hn = r["hnorm"].reshape(T, cpt).copy()
                gap = r["gap"].reshape(T, cpt)
                pages, offs = slots // sc.page_tokens, slots % sc.page_tokens
                ok = (slots >= 0) & (slots < sc.num_pages * sc.page_tokens)   # others are skipped
                if B > 0:
                    for pos, val in zip(r["side_pos"], r["side_val"]):
                        t, c = divmod(int(pos), cpt)
                        if not ok[t]:
                            continue
                        found += 1
                        lst = self.side[l][h][pages[t]]
                        if len(lst) < sc.page_capacity:
                            lst.append((int(offs[t]) * cpt + c, val.copy()))
                        else:
                            hn[t, c] &= 0x7FFF
                            dropped += 1
                for t in np.flatnonzero(ok):
                    self.codes[l, h, pages[t], offs[t]] = codes[t]
                    self.h16[l, h, pages[t], offs[t]] = hn[t]
                    self.gap[l, h, pages[t], offs[t]] = gap[t]
        ok = (slots >= 0) & (slots < sc.num_pages * sc.page_tokens)
        self.written[slots[ok] // sc.page_tokens, slots[ok] % sc.page_tokens] = True
        self.found.append(found)
        self.dropped.append(dropped)


@dataclass
class Replay:
    sc: Scenario
    desc: K.Desc
    pdesc: K.PagedDesc
    pools: dict
    cbh: dict
    cbd: dict
    models: dict
    page_lists: dict      # sequence -> its pages in order
    lengths: dict         # sequence -> tokens
    statuses: list
    guards: list = field(default_factory=list)   # (name, buffer, used bytes) when guarded


GUARD_BYTE = 0xA5


def _guard_pool(pool: K.Pool, role: int, guards: list) -> None:
    """Move every plane of ``pool`` to the front of a buffer whose tail holds
    GUARD_BYTE (page counts start at zero as in a fresh pool)."""
    for name in ("idx", "hnorm", "side_count", "side_pos", "side_val"):
        t = getattr(pool, name)
        nbytes = t.numel() * t.element_size()
        buf = torch.full((nbytes + 4096,), GUARD_BYTE, dtype=torch.uint8, device=t.device)
        view = buf[:nbytes].view(t.dtype).view(t.shape)
        if name == "side_count":
            view.zero_()
        setattr(pool, name, view)
        setattr(pool.c, name, buf.data_ptr())
        guards.append((f"role {role} {name}", buf, nbytes))


def replay(sc: Scenario, guard: bool = False) -> Replay:
    """Run every call on the GPU (K and V pools) and in the model.  guard:
    the pools' planes are followed by patterned bytes (see ``_guard_pool``)."""
    pdesc = _pdesc(sc)
    desc0 = _desc(sc, 0)
    rng = np.random.default_rng(sc.seed)
    free = list(rng.permutation(sc.num_pages))
    page_lists, lengths = {}, {}
    pools, cbh, cbd, models = {}, {}, {}, {}
    for role in (0, 1):
        cbh[role] = K.hqmq_make_codebook(sc.seed, sc.layers, sc.heads, role, sc.S)
        cbd[role] = torch.from_numpy(cbh[role]).cuda()
        pools[role] = K.allocate_pool(desc0, pdesc)
        models[role] = PoolModel(sc, cbh[role])
    statuses = []
    guards = []
    if guard:
        for role in (0, 1):
            _guard_pool(pools[role], role, guards)
    for i, call in enumerate(sc.calls):
        slots = []
        for seq, n in call:
            pl = page_lists.setdefault(seq, [])
            t0 = lengths.get(seq, 0)
            for t in range(t0, t0 + n):
                if t // sc.page_tokens >= len(pl):
                    pl.append(int(free.pop()))
                slots.append(pl[t // sc.page_tokens] * sc.page_tokens + t % sc.page_tokens)
            lengths[seq] = t0 + n
        slots = np.array(slots, np.int64)
        T = len(slots)
        desc = _desc(sc, T)
        sl_dev = torch.from_numpy(slots).cuda()
        st = []
        for role in (0, 1):
            x = _call_input(sc, 2 * i + role, T)
            status = torch.zeros(2, dtype=torch.int64, device="cuda")
            print(f"append call {i} role {role}: {T} tokens", flush=True)
            K.append(desc, pdesc, pools[role], x, sl_dev, cbd[role], status=status)
            torch.cuda.synchronize()
            models[role].apply(x.float().cpu().numpy(), slots)
            st.append(status.cpu().numpy().tolist())
        statuses.append(st)
    return Replay(sc, desc0, pdesc, pools, cbh, cbd, models, page_lists, lengths, statuses, guards)


def compare_records(rp: Replay) -> dict:
    """Record differences between the GPU pools and the model: near-tie codes
    (allowed) and everything else (must be 0)."""
    sc = rp.sc
    cpt = sc.head_dim // 4
    b = O.code_bits(sc.S)
    rep = {"near_tie_codes": 0, "mismatch": 0, "rows": 0, "entries": 0, "status_mismatch": 0}
    for i, st in enumerate(rp.statuses):
        for role in (0, 1):
            m = rp.models[role]
            if st[role] != [m.found[i], m.dropped[i]]:
                rep["status_mismatch"] += 1
    for role in (0, 1):
        m, pool = rp.models[role], rp.pools[role]
        idx = pool.idx.cpu().numpy().view(np.uint32)
        hn = pool.hnorm.cpu().numpy()
        count = pool.side_count.cpu().numpy().view(np.uint32)
        spos = pool.side_pos.cpu().numpy().view(np.uint32)
        sval = pool.side_val.cpu().numpy().view(np.uint16)
        w = m.written
        codes_g = P.unpack_words(idx[:, :, w], cpt, b)                # [L, H, rows, cpt]
        codes_o = m.codes[:, :, w]
        diff = codes_g != codes_o
        near = diff & (m.gap[:, :, w] < P.GAP_EXEMPT)
        rep["near_tie_codes"] += int(near.sum())
        rep["mismatch"] += int((diff & ~near).sum())
        if sc.norm_format == K.HQMQ_NORM_PACKED:
            nc_g = P.unpack_words(hn.view(np.uint32)[:, :, w], cpt, b)
            rep["mismatch"] += int((nc_g != O.compact_norms(m.h16[:, :, w], b)).sum())
        else:
            rep["mismatch"] += int((hn.view(np.uint16)[:, :, w] != m.h16[:, :, w]).sum())
        rep["rows"] += int(w.sum()) * sc.layers * sc.heads
        # side lists of every page
        for l in range(sc.layers):
            for h in range(sc.heads):
                for pg in range(sc.num_pages):
                    want = m.side[l][h][pg]
                    n = int(count[l, h, pg])
                    if n != len(want):
                        rep["mismatch"] += abs(n - len(want)) + 1
                        continue
                    rep["entries"] += n
                    for k, (pos, val) in enumerate(want):
                        if spos[l, h, pg, k] != pos or np.any(sval[l, h, pg, k] != val):
                            rep["mismatch"] += 1
        # the decoded values use the GPU's code where a near tie let it differ
        codes_used = m.codes.copy()
        cu = codes_used[:, :, w]
        cu[near] = codes_g[near]
        codes_used[:, :, w] = cu
        m.codes_used = codes_used
    return rep


def decoded_sequence(rp: Replay, role: int, l: int, h: int, seq: int) -> np.ndarray:
    """The model's binary16 decoded values of sequence seq in slice (l, h)."""
    sc = rp.sc
    m = rp.models[role]
    cpt = sc.head_dim // 4
    n = rp.lengths[seq]
    rows = []
    for j, pg in enumerate(rp.page_lists[seq]):
        used = min(sc.page_tokens, n - j * sc.page_tokens)
        if used <= 0:
            break
        codes = m.codes_used[l, h, pg, :used].reshape(-1)
        hn = m.h16[l, h, pg, :used].reshape(-1)
        if sc.norm_format == K.HQMQ_NORM_PACKED:
            hn = O.compact_to_h16(O.compact_norms(hn, O.code_bits(sc.S)), O.code_bits(sc.S))
        lst = [e for e in m.side[l][h][pg] if e[0] < used * cpt]
        pos = np.array([e[0] for e in lst], np.uint32) if lst else None
        val = np.array([e[1] for e in lst], np.uint16).reshape(-1, 4) if lst else None
        y = O.decode_range(codes, hn, used, sc.head_dim, m.cb[l, h], pos, val, 0)
        rows.append(A.f16_values(y))
    return np.concatenate(rows) if rows else np.zeros((0, sc.head_dim))


def attend_case(rp: Replay, group: int, scale: float, seqs=None, max_len=None, extra_pages: int = 0,
                seed: int = 0) -> float:
    """Attention over the pools for the given sequences (default: all), every
    layer; returns the worst error / tolerance ratio."""
    sc = rp.sc
    if not all(hasattr(m, "codes_used") for m in rp.models.values()):
        rep = compare_records(rp)   # also settles the codes the decoded values use
        assert rep["mismatch"] == 0, rep
    seqs = sorted(rp.lengths) if seqs is None else seqs
    lens = [rp.lengths[s] for s in seqs]
    maxp = max([len(rp.page_lists[s]) for s in seqs] + [1]) + extra_pages
    pt = np.zeros((len(seqs), maxp), np.int32)
    for i, s in enumerate(seqs):
        pt[i, :len(rp.page_lists[s])] = rp.page_lists[s]
    if max_len is None:
        max_len = max(lens + [0])
    q = A.make_queries(len(seqs), sc.heads * group, sc.head_dim, seed)
    qn = q.float().cpu().numpy().astype(np.float64)
    pt_d = torch.from_numpy(pt).cuda()
    sl_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    worst = 0.0
    for l in range(sc.layers):
        out = K.attend_paged(rp.desc, rp.pdesc, l, rp.pools[0], rp.cbd[0], rp.pools[1], rp.cbd[1], q, pt_d,
                             sl_d, max_len, scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for i, s in enumerate(seqs):
            n = min(lens[i], max_len)
            for h in range(sc.heads):
                kk = decoded_sequence(rp, 0, l, h, s)[:n]
                vv = decoded_sequence(rp, 1, l, h, s)[:n]
                ref = O.attend(kk, vv, qn[i, h * group:(h + 1) * group], scale)
                worst = max(worst, A.compare_out(got[i, h * group:(h + 1) * group], ref, vv))
    return worst
