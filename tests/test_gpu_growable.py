"""GPU parity of growable tables: row handles apart from the key index, and
ht_resize, which rehashes only the index (MTGR, arXiv 2505.18654, section 5:
capacity expansion replicates key storage, not the embeddings).

Checked against the oracle (whose resize only raises the FULL bound) and
against fixed tables: statuses, gathered rows bit-exact; row handles stay
valid across a resize; tombstones are dropped; handles of erased keys are
reused; Adam state and last_seen survive a resize.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _keys(rng, n, lo=0, hi=1 << 40):
    return np.unique(rng.integers(lo, hi, n)).astype(np.int64)


def test_growable_forward_matches_fixed_table(htl, orc):
    w = workloads.tiny()
    keys = torch.from_numpy(w.keys).cuda()
    fixed = htl.Table(w.capacity_log2, w.dim, "f32")
    grow = htl.Table(w.capacity_log2, w.dim, "f32", growable=True)
    for _ in range(2):                      # first pass inserts, second finds
        out_f, uniq, inv, nu, _, st_f = htl.lookup(fixed, keys)
        out_g, uniq2, inv2, nu2, slots, st_g = htl.lookup(grow, keys)
        U = int(nu.item())
        assert np.array_equal(to_np(out_f), to_np(out_g))
        assert np.array_equal(np.sort(to_np(uniq)[:U]), np.sort(to_np(uniq2)[:U]))
        assert np.array_equal(np.sort(to_np(st_f)[:U]), np.sort(to_np(st_g)[:U]))
        h = to_np(slots)[:U]
        assert h.min() >= 0 and h.max() < U and np.unique(h).size == U   # fresh table: handles 0..U-1
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.F32)
    otab.find_or_insert(np.unique(w.keys))
    assert np.array_equal(to_np(out_g), otab.gather(w.keys))


def test_resize_keeps_handles_rows_and_state(htl, orc):
    rng = np.random.default_rng(5)
    dim = 8
    table = htl.Table(10, dim, "f32", last_seen=True, adam=True, growable=True)
    otab = orc.Table(1 << 10, dim, orc.F32, adam=True)
    keys = _keys(rng, 900)
    k_d = torch.from_numpy(keys).cuda()
    slots, st = table.find_or_insert(k_d, step=7)
    assert np.all(to_np(st) == htl.INSERTED)
    otab.find_or_insert(keys, step=7)
    gone = keys[::3]
    assert np.all(to_np(table.erase(torch.from_numpy(gone).cuda())) == htl.ERASED)
    otab.erase(gone)
    live = np.setdiff1d(keys, gone)
    l_d = torch.from_numpy(live).cuda()
    h0, st0 = table.find_or_insert(l_d, step=9)
    assert np.all(to_np(st0) == htl.FOUND)
    otab.find_or_insert(live, step=9)
    g = torch.from_numpy(rng.standard_normal((live.size, dim)).astype(np.float32)).cuda()
    htl.rowwise_adam(table, h0, g, None, 1e-3, 0.9, 0.999, 1e-8, 1)
    before = {n: to_np(htl.table_tensor(table, n))[to_np(h0)] for n in ("rows", "adam_m", "adam_v")}
    assert np.count_nonzero(to_np(htl.table_keys(table)) == htl.TOMBSTONE_KEY) == gone.size

    def live_state():
        k, ls, h, n = table.scan()
        L = int(n.item())
        o = np.argsort(to_np(k)[:L])
        return to_np(k)[:L][o], to_np(ls)[:L][o], to_np(h)[:L][o]

    ks0, ls0, hs0 = live_state()
    assert np.array_equal(ks0, live) and np.all(ls0 == 9)

    table.resize(12)
    otab.resize(1 << 12)
    assert table.capacity == 4096
    k_after = to_np(htl.table_keys(table))
    assert np.count_nonzero(k_after == htl.TOMBSTONE_KEY) == 0            # tombstones dropped
    assert np.array_equal(np.sort(k_after[k_after >= 0]), live)
    for n, b in before.items():                                           # rows did not move
        assert np.array_equal(to_np(htl.table_tensor(table, n))[to_np(h0)], b), n
    ks1, ls1, hs1 = live_state()                                          # last_seen moved with its key
    assert np.array_equal(ks1, ks0) and np.array_equal(ls1, ls0) and np.array_equal(hs1, hs0)
    h1, st1 = table.find_or_insert(l_d, step=11)
    assert np.all(to_np(st1) == htl.FOUND)
    assert np.array_equal(to_np(h1), to_np(h0))                           # handles are stable
    # erased keys are absent; re-inserted they get their closed-form rows
    assert np.all(to_np(table.erase(torch.from_numpy(gone).cuda())) == htl.NOT_FOUND)
    h2, st2 = table.find_or_insert(torch.from_numpy(gone).cuda(), step=11)
    assert np.all(to_np(st2) == htl.INSERTED)
    assert np.all(otab.find_or_insert(gone, step=11) == orc.INSERTED)
    assert np.array_equal(to_np(htl.gather(table, h2)), otab.gather(gone))
    # fill to the new capacity, then FULL
    new = _keys(rng, 8000, 1 << 41, 1 << 42)[: 4096 - keys.size]
    h3, st3 = table.find_or_insert(torch.from_numpy(new).cuda())
    assert np.all(to_np(st3) == htl.INSERTED)
    assert to_np(table.find_or_insert(torch.tensor([1 << 43], device="cuda"))[1])[0] == htl.FULL
    allh = np.concatenate([to_np(h1), to_np(h2), to_np(h3)])
    assert np.array_equal(np.sort(allh), np.arange(4096))                 # every handle in use once


def test_erased_handles_are_reused(htl):
    rng = np.random.default_rng(6)
    table = htl.Table(12, 4, "bf16", growable=True)
    keys = _keys(rng, 3000)
    h, _ = table.find_or_insert(torch.from_numpy(keys).cuda())
    freed = set(to_np(h)[:1000].tolist())
    table.erase(torch.from_numpy(keys[:1000]).cuda())
    new = _keys(rng, 2000, 1 << 41, 1 << 42)[:700]
    h2, st = table.find_or_insert(torch.from_numpy(new).cuda())
    assert np.all(to_np(st) == htl.INSERTED)
    assert set(to_np(h2).tolist()) <= freed                               # taken from the free stack
    h3, _ = table.find_or_insert(torch.from_numpy(_keys(rng, 2000, 1 << 42, 1 << 43)[:800]).cuda())
    h3 = to_np(h3)
    assert np.count_nonzero(np.isin(h3, list(freed))) == 300              # the rest of the stack ...
    assert np.all(h3[~np.isin(h3, list(freed))] >= 3000)                 # ... then never-used rows


def test_duplicate_keys_in_one_call_share_a_handle(htl):
    table = htl.Table(10, 4, "f32", growable=True)
    keys = torch.tensor([5, 9, 5, 5, 9, 12], dtype=torch.int64, device="cuda")
    h, st = table.find_or_insert(keys)
    h, st = to_np(h), to_np(st)
    for k in (5, 9):
        idx = np.flatnonzero(to_np(keys) == k)
        assert np.unique(h[idx]).size == 1
        assert np.count_nonzero(st[idx] == htl.INSERTED) == 1


def test_backward_on_growable_matches_fixed(htl):
    rng = np.random.default_rng(7)
    n, dim = 1 << 14, 32
    keys_np = workloads.backward(n=n, dim=4, with_grad=False).keys
    keys = torch.from_numpy(keys_np).cuda()
    grad = torch.from_numpy((rng.integers(-8, 9, (n, dim)) * 2.0 ** -6).astype(np.float32)).cuda()
    res = []
    for growable in (False, True):
        t = htl.Table(15, dim, "f32", adam=True, growable=growable)
        uniq, inv, nu = htl.dedup_unique_inverse(keys, ordered=True)
        slots, _ = t.find_or_insert(uniq, n_dev=nu)
        htl.segment_sum_adam(t, slots, grad, inv, nu, n)
        U = int(nu.item())
        res.append(to_np(htl.gather(t, slots[:U])))
    assert np.array_equal(res[0].view(np.uint32), res[1].view(np.uint32))


def test_resize_errors(htl):
    fixed = htl.Table(8, 4, "f32")
    with pytest.raises(htl.HTLError):
        fixed.resize(9)
    grow = htl.Table(8, 4, "f32", growable=True)
    with pytest.raises(htl.HTLError):
        grow.resize(7)                     # shrinking
    with pytest.raises(htl.HTLError):
        grow.resize(17)                    # beyond the reservation (created + 8)
    grow.resize(8)                         # same size: a rehash
    grow.resize(16)
    assert grow.capacity == 1 << 16
