"""GPU parity of the fused forward entry point ht_lookup.

ht_lookup must produce what dedup_unique_inverse + ht_find_or_insert +
emb_gather_pool produce: the same unique-key set, the same ID -> key map,
the same status per key and the same rows, bit for bit -- only the order of
the unique keys differs (slot order).  It also keeps a per-slot touch map in
the table that must be all zero after every call, which the repeated-call
tests check indirectly (a dirty map would add phantom unique keys).
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _fused_parity(htl, orc, table, otab, keys_np, step=0, full_ok=False):
    keys = torch.from_numpy(keys_np).cuda()
    out, uniq, inv, nu, slots, status = table.lookup(keys, step=step, phases=bool(step % 2))
    U = int(nu.item())
    u, st, sl, iv = to_np(uniq)[:U], to_np(status)[:U], to_np(slots)[:U], to_np(inv)
    ref_u, _ = orc.dedup(keys_np)
    assert U == ref_u.size
    assert np.array_equal(np.sort(u), ref_u)
    if keys_np.size:
        assert iv.min() >= 0 and iv.max() < U
        assert np.array_equal(u[iv], keys_np)
    if full_ok:
        order = np.argsort(st == htl.FULL, kind="stable")
        ref_st = np.empty_like(st)
        ref_st[order] = otab.find_or_insert(u[order], step=step)
    else:
        ref_st = otab.find_or_insert(u, step=step)
    assert np.array_equal(st, ref_st)
    ok = st <= 1
    assert np.all(sl[ok] >= 0) and np.unique(sl[ok]).size == int(ok.sum())
    assert np.all(sl[~ok] == -1)
    assert np.array_equal(to_np(out), otab.gather(keys_np))
    return u, st, sl


def test_fused_tiny_twice(htl, orc):
    w = workloads.tiny()
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    otab = orc.Table(1 << w.capacity_log2, w.dim)
    u, st, sl = _fused_parity(htl, orc, table, otab, w.keys)
    assert np.all(st == htl.INSERTED)
    u2, st2, sl2 = _fused_parity(htl, orc, table, otab, w.keys, step=1)
    assert np.all(st2 == htl.FOUND)
    assert dict(zip(u.tolist(), sl.tolist())) == dict(zip(u2.tolist(), sl2.tolist()))
    # slot order: unique keys come out sorted by slot
    assert np.all(np.diff(sl2) > 0)


@pytest.mark.parametrize("dim,dtype", [(64, "f32"), (128, "bf16"), (16, "f32"), (3, "f32"), (5, "bf16"),
                                       (200, "f32")])
def test_fused_row_shapes(htl, orc, dim, dtype):
    rng = np.random.default_rng(dim)
    keys = rng.integers(0, 5000, 30000).astype(np.int64) << np.int64(20)
    table = htl.Table(14, dim, dtype, init_seed=dim)
    otab = orc.Table(1 << 14, dim, orc.F32 if dtype == "f32" else orc.BF16, seed=dim)
    _fused_parity(htl, orc, table, otab, keys)


@pytest.mark.parametrize("n", [1, 2047, 2048, 2049, 70001])
def test_fused_sizes_and_prefill(htl, orc, n):
    w = workloads.single_large_table(n=n, capacity_log2=16, prefill_count=1 << 14, universe_log2=20)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    otab = orc.Table(1 << w.capacity_log2, w.dim)
    table.find_or_insert(torch.from_numpy(w.prefill).cuda())
    otab.find_or_insert(w.prefill)
    for step in range(3):
        _fused_parity(htl, orc, table, otab, w.keys, step=step)


def test_fused_reserved_and_special_keys(htl, orc):
    i64 = np.iinfo(np.int64)
    rng = np.random.default_rng(3)
    base = np.array([-1, -2, i64.min, i64.max, 0, 7], dtype=np.int64)
    keys = np.concatenate([rng.choice(base, 9000), rng.integers(0, 3000, 9000)]).astype(np.int64)
    rng.shuffle(keys)
    table = htl.Table(13, 8, "f32")
    otab = orc.Table(1 << 13, 8)
    u, st, sl = _fused_parity(htl, orc, table, otab, keys)
    assert set(u[st == htl.RESERVED].tolist()) == {-1, -2}


def test_fused_table_runs_full(htl, orc):
    # 4096 slots, ~6000 distinct keys: the spill path gives FULL keys their ids
    rng = np.random.default_rng(11)
    table = htl.Table(12, 4, "f32")
    otab = orc.Table(1 << 12, 4)
    for rnd in range(3):
        keys = rng.integers(0, 6000 + rnd * 1000, 20000).astype(np.int64)
        u, st, sl = _fused_parity(htl, orc, table, otab, keys, step=rnd, full_ok=True)
        assert (st == htl.FULL).any()
    # once the table is full, only live keys are FOUND; a later call without
    # FULL keys must still be exact (the spill path leaves nothing behind)
    live, _ = otab.live()
    _fused_parity(htl, orc, table, otab, live[:3000], step=9)


def test_fused_matches_separate_path(htl, orc):
    w = workloads.single_large_table(n=1 << 17, capacity_log2=19, prefill_count=1 << 18)
    pre = torch.from_numpy(w.prefill).cuda()
    keys = torch.from_numpy(w.keys).cuda()
    a = htl.Table(w.capacity_log2, w.dim, w.dtype)
    b = htl.Table(w.capacity_log2, w.dim, w.dtype)
    a.find_or_insert(pre)
    b.find_or_insert(pre)
    out_a, ua, ia, na, sa, sta = a.lookup(keys)
    out_b, ub, ib, nb, sb, stb = htl.lookup(b, keys)
    U = int(na.item())
    assert U == int(nb.item())
    ka = dict(zip(to_np(ua)[:U].tolist(), to_np(sta)[:U].tolist()))
    kb = dict(zip(to_np(ub)[:U].tolist(), to_np(stb)[:U].tolist()))
    assert ka == kb
    assert torch.equal(out_a, out_b)
    assert torch.equal(ua[ia.long()], ub[ib.long()])


def test_fused_last_seen_and_erase(htl, orc):
    rng = np.random.default_rng(5)
    table = htl.Table(12, 8, "bf16", last_seen=True)
    otab = orc.Table(1 << 12, 8, orc.BF16)
    for step in range(6):
        keys = rng.integers(0, 2500, 8000).astype(np.int64)
        _fused_parity(htl, orc, table, otab, keys, step=step)
        er = np.unique(rng.integers(0, 2500, 700)).astype(np.int64)
        assert np.array_equal(to_np(table.erase(torch.from_numpy(er).cuda())), otab.erase(er))
    lk, ls, _, n = table.scan()
    L = int(n.item())
    order = np.argsort(to_np(lk)[:L])
    ref_k, ref_ls = otab.live()
    assert np.array_equal(to_np(lk)[:L][order], ref_k)
    assert np.array_equal(to_np(ls)[:L][order].astype(np.uint32), ref_ls)


def test_fused_empty_batch(htl, orc):
    table = htl.Table(8, 4, "f32")
    out, uniq, inv, nu, slots, status = table.lookup(torch.empty(0, dtype=torch.int64, device="cuda"))
    assert int(nu.item()) == 0 and out.shape == (0, 4)


@pytest.mark.slow
def test_fused_single_large_table_full_size(htl, orc):
    w = workloads.single_large_table()
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    _, st = table.find_or_insert(torch.from_numpy(w.prefill).cuda())
    assert bool((st == htl.INSERTED).all())
    keys = torch.from_numpy(w.keys).cuda()
    for step in range(2):
        out, uniq, inv, nu, slots, status = table.lookup(keys, step=step)
        U = int(nu.item())
        u = to_np(uniq)[:U]
        assert np.array_equal(np.sort(u), np.unique(w.keys))
        assert np.array_equal(u[to_np(inv)], w.keys)
        stn = to_np(status)[:U]
        expect_found = np.isin(u, w.prefill) if step == 0 else np.ones(U, bool)
        assert np.array_equal(stn == htl.FOUND, expect_found)
        assert np.all(stn <= 1)
        rng = np.random.default_rng(step)
        idx = np.concatenate([rng.integers(0, w.keys.size, 4096), [0, w.keys.size - 1]])
        got = to_np(out[torch.from_numpy(idx).cuda()])
        assert np.array_equal(got, orc.init_rows(w.keys[idx], w.dim, orc.F32))
