"""GPU parity of the online-table steps: find-or-insert with a step stamp,
gather, least-recently-used victim choice, and erase -- over a drifting
Zipf stream, step by step against the oracle.

Victim sets are compared as sets (their order is unspecified); statuses per
key, live key sets with their last_seen, and gathered bf16 rows bit-exact.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _run_online(htl, orc, spec, steps, growable=False, grow_at=()):
    table = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, growable=growable)
    otab = orc.Table(1 << spec.capacity_log2, spec.dim, orc.BF16)
    for s in range(steps):
        if s in grow_at:
            table.resize(table.capacity_log2 + 1)
            otab.resize(table.capacity)
        keys_np = workloads.dynamic_online_step(spec, s)
        keys = torch.from_numpy(keys_np).cuda()
        out, uniq, inv, nu, slots, status = htl.lookup(table, keys, step=s)
        U = int(nu.item())
        u = to_np(uniq)[:U]
        assert np.array_equal(to_np(status)[:U], otab.find_or_insert(u, step=s))
        assert np.array_equal(to_np(out), otab.gather(keys_np))
        victims, nv = table.lru_select(spec.evict_num, spec.evict_den)
        k = int(nv.item())
        ref_v = otab.lru_victims(spec.evict_num, spec.evict_den)
        assert k == ref_v.size
        assert np.array_equal(np.sort(to_np(victims)[:k]), np.sort(ref_v))
        st = table.erase(victims[:k])
        assert np.all(to_np(st) == htl.ERASED)
        otab.erase(ref_v)
        lk, ls, sl, n = table.scan()
        L = int(n.item())
        assert L == len(otab)
        order = np.argsort(to_np(lk)[:L])
        ref_k, ref_ls = otab.live()
        assert np.array_equal(to_np(lk)[:L][order], ref_k)
        assert np.array_equal(to_np(ls)[:L][order].astype(np.uint32), ref_ls)


def test_online_small(htl, orc):
    spec = workloads.DynamicOnlineSpec(window=1 << 14, n=1 << 12, capacity_log2=16, dim=64)
    _run_online(htl, orc, spec, steps=8)


def test_online_heavy_eviction(htl, orc):
    spec = workloads.DynamicOnlineSpec(window=1 << 12, n=1 << 11, capacity_log2=13, dim=8,
                                       evict_num=1, evict_den=3)
    _run_online(htl, orc, spec, steps=6)


def test_online_growable_with_resizes(htl, orc):
    """The same stream on a growable table (row handles, rows apart from the
    key index), grown twice mid-stream: every status, gathered row, victim
    set and live set still matches the oracle."""
    spec = workloads.DynamicOnlineSpec(window=1 << 14, n=1 << 12, capacity_log2=14, dim=64)
    _run_online(htl, orc, spec, steps=8, growable=True, grow_at=(3, 6))


def test_online_growable_heavy_eviction(htl, orc):
    spec = workloads.DynamicOnlineSpec(window=1 << 12, n=1 << 11, capacity_log2=12, dim=8,
                                       evict_num=1, evict_den=3)
    _run_online(htl, orc, spec, steps=6, growable=True, grow_at=(2,))


def test_lru_edge_fractions(htl, orc):
    table = htl.Table(10, 4, "bf16", last_seen=True)
    otab = orc.Table(1 << 10, 4, orc.BF16)
    rng = np.random.default_rng(4)
    for s in range(5):
        ks = np.unique(rng.integers(0, 600, 200)).astype(np.int64)
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=s * 300)   # last_seen above one byte
        otab.find_or_insert(ks, step=s * 300)
    for num, den in ((0, 1), (1, 1), (1, 2), (3, 7), (1, 1000)):
        victims, nv = table.lru_select(num, den)
        k = int(nv.item())
        ref = otab.lru_victims(num, den)
        assert k == ref.size
        assert np.array_equal(np.sort(to_np(victims)[:k]), np.sort(ref))
    # a victim buffer smaller than k holds some of the victims, n reports all
    victims, nv = table.lru_select(1, 2, victims_cap=5)
    ref = otab.lru_victims(1, 2)
    assert int(nv.item()) == ref.size
    assert set(to_np(victims)[:5].tolist()) <= set(ref.tolist())


def test_lru_requires_metadata(htl):
    table = htl.Table(6, 4, "f32")
    with pytest.raises(htl.HTLError):
        table.lru_select(1, 20)


def test_lru_many_ties(htl, orc):
    # 40,000 keys share the newest last_seen, so the victim cut falls inside
    # one last_seen value: the key digits decide, over ties spread across all
    # 16 chunks of 4096 slots; half the keys are small (their top digits all
    # equal), half span the whole signed range
    table = htl.Table(16, 4, "bf16", last_seen=True)
    otab = orc.Table(1 << 16, 4, orc.BF16)
    rng = np.random.default_rng(9)
    old = rng.integers(-(1 << 62), 1 << 62, 10_000).astype(np.int64)
    small = np.arange(20_000, dtype=np.int64)
    wide = rng.integers(-(1 << 63), (1 << 63) - 1, 20_000, dtype=np.int64)
    new = np.unique(np.concatenate([small, wide]))
    old = np.setdiff1d(old, new)
    for ks, step in ((old, 3), (new, 5)):
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=step)
        otab.find_or_insert(ks, step=step)
    for num, den in ((1, 2), (3, 4), (1, 5), (999, 1000)):
        victims, nv = table.lru_select(num, den)
        k = int(nv.item())
        ref = otab.lru_victims(num, den)
        assert k == ref.size
        assert np.array_equal(np.sort(to_np(victims)[:k]), np.sort(ref))


@pytest.mark.parametrize("growable", [False, True])
def test_lru_sees_only_live_slots(htl, orc, growable):
    # erased, cleared and rehashed slots must not be eviction candidates:
    # selecting every live key returns exactly the live set
    table = htl.Table(12, 8, "f32", last_seen=True, growable=growable)
    rng = np.random.default_rng(21)
    keys = np.unique(rng.integers(-(1 << 62), 1 << 62, 1500).astype(np.int64))
    table.find_or_insert(torch.from_numpy(keys).cuda(), step=7)
    gone = keys[::3]
    st = to_np(table.erase(torch.from_numpy(gone).cuda()))
    assert (st == htl.ERASED).all()
    live = np.setdiff1d(keys, gone)

    def all_victims():
        victims, nv = table.lru_select(1, 1)
        k = int(nv.item())
        return np.sort(to_np(victims)[:k])

    assert np.array_equal(all_victims(), live)
    if growable:
        table.resize(13)
        assert np.array_equal(all_victims(), live)
    # re-inserting an erased key makes it a candidate again, with its new step
    table.find_or_insert(torch.from_numpy(gone[:10]).cuda(), step=2)
    victims, nv = table.lru_select(10, live.size + 10)
    assert int(nv.item()) == 10
    assert np.array_equal(np.sort(to_np(victims)[:10]), np.sort(gone[:10]))
    table.clear()
    victims, nv = table.lru_select(1, 1)
    assert int(nv.item()) == 0


def test_reserved_step(htl):
    keys = torch.arange(5, dtype=torch.int64).cuda()
    with pytest.raises(htl.HTLError):
        htl.Table(6, 4, "f32", last_seen=True).find_or_insert(keys, step=0xFFFFFFFF)
    _, st = htl.Table(6, 4, "f32").find_or_insert(keys, step=0xFFFFFFFF)   # no last_seen kept: any step
    assert (to_np(st) == htl.INSERTED).all()


def test_lru_select_extremes(htl, orc):
    # k = 0 (num = 0) selects nothing; num = den selects every live key, in
    # any order; victims_cap below k keeps a subset of the victims
    table = htl.Table(10, 4, "f32", last_seen=True)
    otab = orc.Table(1 << 10, 4, orc.F32)
    rng = np.random.default_rng(5)
    for s in range(4):
        ks = np.unique(rng.integers(-(1 << 40), 1 << 40, 100)).astype(np.int64)
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=s)
        otab.find_or_insert(ks, step=s)
    _, nv = table.lru_select(0, 5)
    assert int(nv.item()) == 0
    victims, nv = table.lru_select(7, 7)
    k = int(nv.item())
    ref = otab.lru_victims(7, 7)
    assert k == ref.size and np.array_equal(np.sort(to_np(victims)[:k]), np.sort(ref))
    victims, nv = table.lru_select(1, 2, victims_cap=10)
    k = int(nv.item())
    assert k == otab.lru_victims(1, 2).size and k > 10
    assert np.isin(to_np(victims)[:10], otab.lru_victims(1, 2)).all()
