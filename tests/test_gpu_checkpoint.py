"""GPU parity of checkpointing through compact key scanning (MTGR, arXiv
2505.18654, section 5): ht_export writes the live entries of slot ranges in
slot order, ht_import restores them.

Checked against the oracle (live keys and last_seen, closed-form and
Adam-updated rows) and by round trips: export -> import into an empty table
(fixed or growable, bigger or equal capacity) -> export again gives the same
state, bit for bit, key by key.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _by_key(ck):
    o = np.argsort(ck["keys"], kind="stable")
    return {k: v[o] for k, v in ck.items()}


def _same_state(a, b):
    a, b = _by_key(a), _by_key(b)
    assert a.keys() == b.keys()
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def _populate(htl, orc, table, otab, seed):
    rng = np.random.default_rng(seed)
    keys = np.unique(rng.integers(-(1 << 62), 1 << 62, 3000)).astype(np.int64)
    for step, part in enumerate(np.array_split(keys, 3)):
        k = torch.from_numpy(part).cuda()
        table.find_or_insert(k, step=step + 1)
        otab.find_or_insert(part, step=step + 1)
    gone = keys[::7]
    table.erase(torch.from_numpy(gone).cuda())
    otab.erase(gone)
    return np.setdiff1d(keys, gone)


@pytest.mark.parametrize("dtype,dim,growable", [("f32", 16, False), ("bf16", 64, False), ("bf16", 6, True),
                                                ("f32", 5, True)])
def test_export_matches_oracle_and_round_trips(htl, orc, dtype, dim, growable):
    table = htl.Table(12, dim, dtype, last_seen=True, growable=growable)
    otab = orc.Table(1 << 12, dim, orc.F32 if dtype == "f32" else orc.BF16)
    live = _populate(htl, orc, table, otab, seed=dim)
    ck = table.checkpoint(chunk_slots=1000)            # ranges that split chunks of 4096
    assert np.array_equal(np.sort(ck["keys"]), live)
    ok, ols = otab.live()
    by = _by_key(ck)
    assert np.array_equal(by["keys"], ok) and np.array_equal(by["last_seen"].astype(np.uint32), ols)
    rows = by["rows"].view(np.uint16) if dtype == "bf16" else by["rows"]
    assert np.array_equal(rows, otab.gather(ok))
    # slot order within the export: slots of the keys are increasing
    full = table.export()
    n = int(full["n"].item())
    keys_arr = to_np(htl.table_keys(table))
    slot_of = {int(k): s for s, k in enumerate(keys_arr) if k not in (htl.EMPTY_KEY, htl.TOMBSTONE_KEY)}
    sl = np.array([slot_of[int(k)] for k in to_np(full["keys"])[:n]])
    assert np.all(np.diff(sl) > 0)
    for growable2, log2 in ((False, 12), (True, 13), (False, 14)):
        t2 = htl.Table(log2, dim, dtype, last_seen=True, growable=growable2)
        st = to_np(t2.restore(ck, chunk=700))
        assert np.all(st == htl.INSERTED)
        _same_state(ck, t2.checkpoint())
        # the restored table behaves like the original: same LRU victims
        v1, n1 = table.lru_select(1, 4)
        v2, n2 = t2.lru_select(1, 4)
        k1 = int(n1.item())
        assert k1 == int(n2.item())
        assert np.array_equal(np.sort(to_np(v1)[:k1]), np.sort(to_np(v2)[:k1]))


def test_export_import_adam_state(htl):
    w = workloads.backward(n=1 << 14, dim=32)
    table = htl.Table(15, 32, "f32", adam=True)
    keys = torch.from_numpy(w.keys).cuda()
    uniq, inv, nu = htl.dedup_unique_inverse(keys)
    slots, _ = table.find_or_insert(uniq, n_dev=nu)
    htl.segment_sum_adam(table, slots, torch.from_numpy(w.grad).cuda(), inv, nu, keys.numel())
    ck = table.checkpoint()
    assert set(ck) == {"keys", "rows", "adam_m", "adam_v"}
    assert np.any(ck["adam_m"] != 0)
    for growable in (False, True):
        t2 = htl.Table(15, 32, "f32", adam=True, growable=growable)
        assert np.all(to_np(t2.restore(ck)) == htl.INSERTED)
        _same_state(ck, t2.checkpoint())


def test_import_overwrites_found_and_reports_full(htl):
    table = htl.Table(4, 4, "f32")                        # 16 slots
    keys = torch.arange(10, dtype=torch.int64, device="cuda") * 3 + 1
    table.find_or_insert(keys)
    new_rows = torch.full((12, 4), 0.5, dtype=torch.float32, device="cuda")
    k2 = torch.cat([keys[:4], torch.arange(100, 108, dtype=torch.int64, device="cuda")])
    st = to_np(table.import_(k2, new_rows))
    assert np.all(st[:4] == htl.FOUND)
    assert np.count_nonzero(st[4:] == htl.INSERTED) == 6 and np.count_nonzero(st[4:] == htl.FULL) == 2
    live = st != htl.FULL
    s, _ = table.find_or_insert(k2[torch.from_numpy(live).cuda()])
    assert np.all(to_np(htl.gather(table, s)) == 0.5)


def test_export_errors_and_empty_ranges(htl):
    table = htl.Table(10, 8, "f32")
    d = table.export(100, 100)
    assert int(d["n"].item()) == 0
    with pytest.raises(htl.HTLError):
        table.export(0, 2048)                              # beyond capacity
    with pytest.raises(htl.HTLError):
        table.export(5, 3)


@pytest.mark.parametrize("growable", [False, True])
def test_scan_lists_live_slots_in_slot_order(htl, growable):
    rng = np.random.default_rng(11)
    table = htl.Table(13, 4, "f32", last_seen=True, growable=growable)
    keys = np.unique(rng.integers(0, 1 << 40, 6000)).astype(np.int64)
    table.find_or_insert(torch.from_numpy(keys).cuda(), step=4)
    table.erase(torch.from_numpy(keys[::5]).cuda())
    k, ls, h, n = table.scan()
    L = int(n.item())
    slots = to_np(htl.table_keys(table))
    live_slots = np.flatnonzero((slots != htl.EMPTY_KEY) & (slots != htl.TOMBSTONE_KEY))
    assert L == live_slots.size
    assert np.array_equal(to_np(k)[:L], slots[live_slots])
    assert np.all(to_np(ls)[:L] == 4)
    want_h = to_np(htl.table_tensor(table, "row_of_slot"))[live_slots] if growable else live_slots
    assert np.array_equal(to_np(h)[:L], want_h)


def test_import_of_reserved_last_seen(htl):
    # 0xFFFFFFFF marks slots without a live key, so an imported stamp of that
    # value is stored as 0xFFFFFFFE and the key stays an eviction candidate
    table = htl.Table(8, 4, "f32", last_seen=True)
    keys = torch.tensor([11, 12, 13], dtype=torch.int64).cuda()
    rows = torch.zeros((3, 4), dtype=torch.float32).cuda()
    ls = torch.tensor([5, -1, -2], dtype=torch.int32).cuda()        # 5, 0xFFFFFFFF, 0xFFFFFFFE
    st = table.import_(keys, rows, last_seen=ls)
    assert (st.cpu().numpy() == htl.INSERTED).all()
    d = table.export()
    n = int(d["n"].item())
    got = dict(zip(d["keys"][:n].cpu().tolist(), (d["last_seen"][:n].cpu().numpy().astype(np.uint32)).tolist()))
    assert got == {11: 5, 12: 0xFFFFFFFE, 13: 0xFFFFFFFE}
    victims, nv = table.lru_select(1, 1)
    assert int(nv.item()) == 3
    victims, nv = table.lru_select(1, 3)
    assert int(nv.item()) == 1 and int(victims[0].item()) == 11
    # ties on 0xFFFFFFFE: the smaller key goes first
    victims, nv = table.lru_select(2, 3)
    assert sorted(victims[:2].cpu().tolist()) == [11, 12]
