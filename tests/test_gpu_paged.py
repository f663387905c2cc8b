"""GPU parity of the paged pool: streaming appends into scattered pages
(records, Med3x flags and per-page side lists bit-exact against a model of
the pool built from the oracle) and attention over the pages (within the
bound of tests/attend_cases.py).  Helpers and the model: tests/paged_cases.py."""
import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_hqmq_amd as K
from tests import paged_cases as PC

pytestmark = pytest.mark.gpu


def _records_ok(rp, label):
    rep = PC.compare_records(rp)
    print(label, rep, rp.statuses, flush=True)
    assert rep["mismatch"] == 0, rep
    assert rep["status_mismatch"] == 0, (rp.statuses, [m.found for m in rp.models.values()])
    return rep


def test_append_prefill_and_decode_steps():
    """Prefills of several lengths (a page and a half, exactly one page, one
    token, none), decode steps of one token per sequence, a sequence that
    starts later: every written row and page list equals the model."""
    rp = PC.replay(PC.Scenario())
    rep = _records_ok(rp, "default")
    assert rep["entries"] > 0


def test_pool_writes_stay_inside_their_planes():
    """The default scenario on pools whose planes are followed by patterned
    bytes: the appends leave every tail unchanged and the records match the
    model."""
    rp = PC.replay(PC.Scenario(seed=3), guard=True)
    torch.cuda.synchronize()
    for name, buf, nbytes in rp.guards:
        assert torch.all(buf[nbytes:] == PC.GUARD_BYTE), f"{name}: written past its end"
    _records_ok(rp, "guarded")


def test_append_drops_entries_past_page_capacity():
    rp = PC.replay(PC.Scenario(page_capacity=3, seed=1, outlier_channels=2))
    _records_ok(rp, "capacity 3")
    assert sum(st[0][1] + st[1][1] for st in rp.statuses) > 0, "no entry was dropped"


def test_attend_paged_over_pages_cut_at_capacity():
    """Attention over pools whose page lists were cut at a capacity of 3
    entries: the kept entries are read, the dropped chunks take their records'
    bulk values (as the model decodes them), for one and four query heads per
    KV head."""
    rp = PC.replay(PC.Scenario(page_capacity=3, seed=1, outlier_channels=2))
    _records_ok(rp, "capacity 3")
    assert sum(st[0][1] + st[1][1] for st in rp.statuses) > 0, "no entry was dropped"
    for group in (4, 1):
        ratio = PC.attend_case(rp, group, 1.0 / math.sqrt(128))
        print("attend paged, capacity 3", group, ratio, flush=True)
        assert ratio <= 1.0


def test_append_packed_norms_and_med3_batches_inside_a_call():
    sc = PC.Scenario(norm_format=K.HQMQ_NORM_PACKED, med_batch_tokens=48, seed=2)
    _records_ok(PC.replay(sc), "packed, B=48")


@pytest.mark.parametrize("P,NP", [(16, 80), (256, 8)])
def test_append_page_sizes(P, NP):
    sc = PC.Scenario(page_tokens=P, num_pages=NP, seed=3)
    sc.calls = [[(0, 300), (1, 17)], [(0, 1), (1, 1), (2, 1)], [(1, 40), (2, 200)]]
    _records_ok(PC.replay(sc), f"P={P}")


def test_append_without_med3_and_skipped_slots():
    """Med3x off (no side lists touched), then a call whose extra tokens have
    slots outside the pool: they are skipped."""
    sc = PC.Scenario(med_batch_tokens=0, head_dim=64, S=8, seed=4)
    rp = PC.replay(sc)
    _records_ok(rp, "no Med3x")
    assert int(rp.pools[0].side_count.sum()) == 0
    # skipped slots (with Med3x on so that their outliers would count)
    sc2 = PC.Scenario(seed=5)
    sc2.calls = [[(0, 70)]]
    rp2 = PC.replay(sc2)
    desc = PC._desc(sc2, 4)
    x = PC._call_input(sc2, 99, 4)
    nslot = sc2.num_pages * sc2.page_tokens
    slot = rp2.page_lists[0][1] * sc2.page_tokens + 6
    slots = np.array([-1, nslot, slot, nslot + 5], np.int64)
    st_call = []
    for role in (0, 1):
        st = torch.zeros(2, dtype=torch.int64, device="cuda")
        K.append(desc, rp2.pdesc, rp2.pools[role], x, torch.from_numpy(slots).cuda(), rp2.cbd[role], status=st)
        torch.cuda.synchronize()
        rp2.models[role].apply(x.float().cpu().numpy(), slots)
        st_call.append(st.cpu().numpy().tolist())
    rp2.statuses.append(st_call)
    _records_ok(rp2, "skipped slots")


def test_clear_empties_listed_pages_only():
    rp = PC.replay(PC.Scenario(seed=6))
    pool = rp.pools[0]
    before = pool.side_count.clone()
    pages = torch.tensor(rp.page_lists[0] + [-3, 10 ** 6], dtype=torch.int32, device="cuda")
    K.hqmq_paged_clear(rp.desc, rp.pdesc, pool, pages)
    torch.cuda.synchronize()
    after = pool.side_count
    mask = torch.zeros(rp.sc.num_pages, dtype=torch.bool, device="cuda")
    mask[rp.page_lists[0]] = True
    assert bool((after[:, :, mask] == 0).all())
    assert torch.equal(after[:, :, ~mask], before[:, :, ~mask])


@pytest.mark.parametrize("group", [4, 1, 16])
def test_attend_paged(group):
    rp = PC.replay(PC.Scenario(seed=7))
    _records_ok(rp, "attend records")
    ratio = PC.attend_case(rp, group, 1.0 / math.sqrt(128))
    print("attend paged", group, ratio, flush=True)
    assert ratio <= 1.0


def test_attend_paged_clips_and_spare_table_entries():
    """max_len below some lengths, page-table rows longer than needed, an
    empty sequence in the batch."""
    sc = PC.Scenario(seed=8)
    sc.calls = [[(0, 150), (1, 64), (2, 3)]]
    rp = PC.replay(sc)
    rp.lengths[3] = 0
    rp.page_lists[3] = []
    assert PC.attend_case(rp, 4, 0.1, max_len=100, extra_pages=2) <= 1.0


def test_attend_paged_packed_and_small_heads():
    sc = PC.Scenario(norm_format=K.HQMQ_NORM_PACKED, seed=9)
    rp = PC.replay(sc)
    _records_ok(rp, "packed attend")
    assert PC.attend_case(rp, 4, 1.0 / math.sqrt(128)) <= 1.0
    sc = PC.Scenario(head_dim=64, S=8, med_batch_tokens=0, page_tokens=32, num_pages=40, seed=10)
    rp = PC.replay(sc)
    assert PC.attend_case(rp, 2, 0.125) <= 1.0


def test_paged_matches_contiguous_attention():
    """The same tokens appended in one call per sequence (Med3x batch = the
    call) and encoded as one contiguous tensor per sequence give the same
    attention output bit for bit when the split plans agree."""
    sc = PC.Scenario(seed=11)
    sc.calls = [[(0, 256)]]
    rp = PC.replay(sc)
    x = {r: PC._call_input(sc, r, 256) for r in (0, 1)}
    desc = PC._desc(sc, 256)
    recs = {r: K.encode(desc, x[r], rp.cbd[r]) for r in (0, 1)}
    q = PC.A.make_queries(1, sc.heads * 4, 128, 3)
    for l in range(sc.layers):
        a = K.attend(desc, l, recs[0], rp.cbd[0], recs[1], rp.cbd[1], q,
                     torch.zeros(1, dtype=torch.int64, device="cuda"),
                     torch.full((1,), 256, dtype=torch.int32, device="cuda"), 256)
        pt = torch.tensor([rp.page_lists[0]], dtype=torch.int32, device="cuda")
        b = K.attend_paged(rp.desc, rp.pdesc, l, rp.pools[0], rp.cbd[0], rp.pools[1], rp.cbd[1], q, pt,
                           torch.full((1,), 256, dtype=torch.int32, device="cuda"), 256)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
