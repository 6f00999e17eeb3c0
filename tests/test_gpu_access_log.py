"""GPU parity of the eviction choice on tables that keep an access log.

With HT_META_ACCESS_LOG, ht_lru_select takes the cut step from the log's
per-step live counts and its candidates from the ring entries of the
oldest steps, instead of reading last_seen of every slot.  Its victims must
be exactly the oracle's -- the floor(live * num / den) live keys smallest
by (last_seen, key) -- at every step of a drifting stream, and also after
each event that ends the log (import, resize, a step going back, an insert
at a step an erase already saw, a full ring, a step span past the records),
when the selection falls back to the scan.  ht_access_log_state tells which
of the two ran.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _serves(table) -> bool:
    return int(table.access_log_state()[0].item()) == 1


def _check_select(htl, table, otab, num, den):
    victims, nv = table.lru_select(num, den)
    k = int(nv.item())
    ref = otab.lru_victims(num, den)
    assert k == ref.size
    assert np.array_equal(np.sort(to_np(victims)[:k]), np.sort(ref))
    return victims, k, ref


def _check_live(table, otab):
    lk, ls, _, n = table.scan()
    L = int(n.item())
    assert L == len(otab)
    order = np.argsort(to_np(lk)[:L])
    ref_k, ref_ls = otab.live()
    assert np.array_equal(to_np(lk)[:L][order], ref_k)
    assert np.array_equal(to_np(ls)[:L][order].astype(np.uint32), ref_ls)


def _run_stream(htl, orc, spec, steps, fused=False, growable=False, grow_at=()):
    table = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, growable=growable, access_log=True)
    otab = orc.Table(1 << spec.capacity_log2, spec.dim, orc.BF16)
    for s in range(steps):
        if s in grow_at:
            table.resize(table.capacity_log2 + 1)
            otab.resize(table.capacity)
        keys_np = workloads.dynamic_online_step(spec, s)
        out, uniq, inv, nu, slots, status = htl.lookup(table, torch.from_numpy(keys_np).cuda(), step=s, fused=fused)
        U = int(nu.item())
        assert np.array_equal(to_np(status)[:U], otab.find_or_insert(to_np(uniq)[:U], step=s))
        assert np.array_equal(to_np(out), otab.gather(keys_np))
        assert _serves(table) == (not grow_at or s < min(grow_at))
        victims, k, ref = _check_select(htl, table, otab, spec.evict_num, spec.evict_den)
        st = table.erase(victims[:k])
        assert np.all(to_np(st) == htl.ERASED)
        otab.erase(ref)
        _check_live(table, otab)
    return table


@pytest.mark.parametrize("fused", [False, True])
def test_log_stream(htl, orc, fused):
    spec = workloads.DynamicOnlineSpec(window=1 << 14, n=1 << 12, capacity_log2=17, dim=16)
    table = _run_stream(htl, orc, spec, steps=10, fused=fused)
    st = to_np(table.access_log_state())
    assert st[0] == 1 and st[1] >= st[2] and st[3] <= 9


def test_log_heavy_eviction(htl, orc):
    # a third of the live keys go every step: the cut step moves fast and the
    # tail with it
    spec = workloads.DynamicOnlineSpec(window=1 << 12, n=1 << 11, capacity_log2=15, dim=8,
                                       evict_num=1, evict_den=3)
    _run_stream(htl, orc, spec, steps=12)


def test_log_growable_until_resize(htl, orc):
    # row handles instead of slots while the log serves; the resize moves keys
    # to new slots, so the log stops and the scan takes over
    spec = workloads.DynamicOnlineSpec(window=1 << 14, n=1 << 12, capacity_log2=16, dim=16)
    _run_stream(htl, orc, spec, steps=7, growable=True, grow_at=(4,))


def test_log_same_step_calls_and_fractions(htl, orc):
    # several calls per step (keys found again in the same step keep their one
    # entry), steps above one byte, and every fraction, including none and all
    table = htl.Table(16, 4, "bf16", last_seen=True, access_log=True)
    otab = orc.Table(1 << 16, 4, orc.BF16)
    rng = np.random.default_rng(4)
    for s in range(6):
        for _ in range(3):
            ks = np.unique(rng.integers(0, 2500, 400)).astype(np.int64)
            table.find_or_insert(torch.from_numpy(ks).cuda(), step=s * 300)
            otab.find_or_insert(ks, step=s * 300)
    assert _serves(table)
    for num, den in ((0, 1), (1, 1000), (1, 7), (1, 2), (3, 4), (1, 1)):
        _check_select(htl, table, otab, num, den)
    assert _serves(table)
    # evict a half, then keep going: the counts follow the erase
    victims, k, ref = _check_select(htl, table, otab, 1, 2)
    table.erase(victims[:k])
    otab.erase(ref)
    ks = np.unique(rng.integers(0, 5000, 800)).astype(np.int64)
    table.find_or_insert(torch.from_numpy(ks).cuda(), step=2000)
    otab.find_or_insert(ks, step=2000)
    for num, den in ((1, 3), (2, 3), (1, 1)):
        _check_select(htl, table, otab, num, den)
    assert _serves(table)
    _check_live(table, otab)


def test_log_ties_on_the_cut_step(htl, orc):
    # 40,000 keys share the newest step: the cut falls inside it and the key
    # digits decide, small keys (top digits equal) and keys over the whole range
    table = htl.Table(18, 4, "bf16", last_seen=True, access_log=True)
    otab = orc.Table(1 << 18, 4, orc.BF16)
    rng = np.random.default_rng(9)
    old = rng.integers(-(1 << 62), 1 << 62, 10_000).astype(np.int64)
    new = np.unique(np.concatenate([np.arange(20_000, dtype=np.int64),
                                    rng.integers(-(1 << 63), (1 << 63) - 1, 20_000, dtype=np.int64)]))
    old = np.setdiff1d(old, new)
    for ks, step in ((old, 3), (new, 5)):
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=step)
        otab.find_or_insert(ks, step=step)
    for num, den in ((1, 2), (3, 4), (1, 5), (999, 1000)):
        _check_select(htl, table, otab, num, den)
    assert _serves(table)


def _filled(htl, orc, capacity_log2=16, n_steps=3, per_step=900, seed=0):
    table = htl.Table(capacity_log2, 4, "bf16", last_seen=True, access_log=True)
    otab = orc.Table(1 << capacity_log2, 4, orc.BF16)
    rng = np.random.default_rng(seed)
    for s in range(n_steps):
        ks = np.unique(rng.integers(0, 4 * per_step, per_step)).astype(np.int64)
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=10 + s)
        otab.find_or_insert(ks, step=10 + s)
    return table, otab, rng


def test_log_ends_on_import(htl, orc):
    table, otab, rng = _filled(htl, orc)
    assert _serves(table)
    ks = np.setdiff1d(np.unique(rng.integers(10_000, 20_000, 500)), otab.live()[0]).astype(np.int64)
    ls = rng.integers(0, 30, ks.size).astype(np.int32)
    rows = torch.zeros((ks.size, 4), dtype=torch.bfloat16, device="cuda")
    table.import_(torch.from_numpy(ks).cuda(), rows, last_seen=torch.from_numpy(ls).cuda())
    for v in np.unique(ls):
        otab.find_or_insert(ks[ls == v], step=int(v))
    assert not _serves(table)
    for num, den in ((1, 4), (1, 2)):
        _check_select(htl, table, otab, num, den)
    # ht_clear starts the log again
    table.clear()
    otab = orc.Table(1 << 16, 4, orc.BF16)
    assert _serves(table)
    ks = np.arange(3000, dtype=np.int64) * 7
    table.find_or_insert(torch.from_numpy(ks).cuda(), step=1)
    otab.find_or_insert(ks, step=1)
    _check_select(htl, table, otab, 1, 3)
    assert _serves(table)


def test_log_ends_when_steps_go_back(htl, orc):
    table, otab, rng = _filled(htl, orc)
    ks = np.unique(rng.integers(0, 8000, 700)).astype(np.int64)
    table.find_or_insert(torch.from_numpy(ks).cuda(), step=5)      # below step 12
    otab.find_or_insert(ks, step=5)
    assert not _serves(table)
    _check_select(htl, table, otab, 1, 3)


def test_log_ends_on_insert_at_the_erase_step(htl, orc):
    table, otab, rng = _filled(htl, orc)
    victims, k, ref = _check_select(htl, table, otab, 1, 3)
    table.erase(victims[:k])
    otab.erase(ref)
    # the same step again after an erase: freed slots may be claimed anew
    ks = np.unique(rng.integers(0, 8000, 700)).astype(np.int64)
    table.find_or_insert(torch.from_numpy(ks).cuda(), step=12)
    otab.find_or_insert(ks, step=12)
    assert not _serves(table)
    _check_select(htl, table, otab, 1, 3)
    _check_live(table, otab)


def test_log_erase_then_next_step_keeps_serving(htl, orc):
    table, otab, rng = _filled(htl, orc)
    for s in range(13, 17):
        victims, k, ref = _check_select(htl, table, otab, 1, 4)
        table.erase(victims[:k])
        otab.erase(ref)
        ks = np.unique(rng.integers(0, 8000, 900)).astype(np.int64)
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=s)
        otab.find_or_insert(ks, step=s)
        assert _serves(table)
    _check_live(table, otab)


def test_log_ends_when_the_ring_fills(htl, orc):
    # 2^14 slots keep a ring of 4096 entries: two steps of ~2900 keys with no
    # eviction between them overrun it
    table = htl.Table(14, 4, "bf16", last_seen=True, access_log=True)
    otab = orc.Table(1 << 14, 4, orc.BF16)
    rng = np.random.default_rng(2)
    for s in range(2):
        ks = np.unique(rng.integers(0, 1 << 40, 2900)).astype(np.int64)
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=s)
        otab.find_or_insert(ks, step=s)
    assert not _serves(table)
    for num, den in ((1, 3), (1, 1)):
        _check_select(htl, table, otab, num, den)


def test_log_ends_when_steps_span_too_far(htl, orc):
    # live keys 70,000 steps apart: more than the 4096 step records
    table, otab, rng = _filled(htl, orc)
    ks = np.arange(50_000, 50_500, dtype=np.int64)
    table.find_or_insert(torch.from_numpy(ks).cuda(), step=70_000)
    otab.find_or_insert(ks, step=70_000)
    assert not _serves(table)
    _check_select(htl, table, otab, 1, 2)


def test_log_ring_reused_over_many_steps(htl, orc):
    # many more entries than the ring holds pass through it, with eviction
    # every step keeping the live steps inside it
    table = htl.Table(14, 4, "bf16", last_seen=True, access_log=True)
    otab = orc.Table(1 << 14, 4, orc.BF16)
    rng = np.random.default_rng(6)
    for s in range(40):
        ks = np.unique(rng.integers(s * 300, s * 300 + 3000, 600)).astype(np.int64)
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=s)
        otab.find_or_insert(ks, step=s)
        victims, k, ref = _check_select(htl, table, otab, 1, 3)
        table.erase(victims[:k])
        otab.erase(ref)
        assert _serves(table)
    st = to_np(table.access_log_state())
    assert st[1] > 4 * 4096          # the ring has wrapped several times
    _check_live(table, otab)


@pytest.mark.parametrize("access_log", [False, True])
def test_cut_among_keys_that_share_high_bits(htl, orc, access_log):
    # keys (table << 48) | id: the ties differ from bit 52 down, so the cut
    # key's first window (20 bits from there) leaves one table's ties -- up to
    # 30,000, more than the final rank holds in LDS -- for its radix passes
    table = htl.Table(19, 4, "bf16", last_seen=True, access_log=access_log)
    otab = orc.Table(1 << 19, 4, orc.BF16)
    rng = np.random.default_rng(12)
    old = (np.arange(8, dtype=np.int64)[:, None] << 48 | rng.integers(0, 1 << 30, (8, 2000))).ravel()
    new = (np.arange(26, dtype=np.int64)[:, None] << 48 | rng.integers(0, 30_000, (26, 3000))).ravel()
    dense = np.arange(30_000, dtype=np.int64) | (3 << 48)               # one table dense in [0, 30000)
    new = np.unique(np.concatenate([new, dense]))
    old = np.unique(old)
    old = np.setdiff1d(old, new)
    for ks, step in ((old, 1), (new, 2)):
        table.find_or_insert(torch.from_numpy(ks).cuda(), step=step)
        otab.find_or_insert(ks, step=step)
    for num, den in ((1, 5), (1, 3), (1, 2), (2, 3), (99, 100)):
        _check_select(htl, table, otab, num, den)
    if access_log:
        assert _serves(table)


def _continue_stream(htl, orc, table, otab, spec, steps):
    for s in steps:
        keys_np = workloads.dynamic_online_step(spec, s)
        out, uniq, inv, nu, slots, status = htl.lookup(table, torch.from_numpy(keys_np).cuda(), step=s)
        U = int(nu.item())
        assert np.array_equal(to_np(status)[:U], otab.find_or_insert(to_np(uniq)[:U], step=s))
        assert _serves(table)
        victims, k, ref = _check_select(htl, table, otab, spec.evict_num, spec.evict_den)
        table.erase(victims[:k])
        otab.erase(ref)
    _check_live(table, otab)


def test_log_rebuilt_after_a_checkpoint_restore(htl, orc):
    # a stream, a checkpoint, the restore into a fresh logged table (which
    # ends its log), the rebuild, and the stream going on with the log serving
    spec = workloads.DynamicOnlineSpec(window=1 << 13, n=1 << 12, capacity_log2=16, dim=8)
    src = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, access_log=True)
    otab = orc.Table(1 << spec.capacity_log2, spec.dim, orc.BF16)
    _continue_stream(htl, orc, src, otab, spec, range(5))
    ck = src.checkpoint()
    dst = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, access_log=True)
    dst.restore(ck)
    assert not _serves(dst)
    _check_select(htl, dst, otab, spec.evict_num, spec.evict_den)    # the scan, exact
    dst.rebuild_access_log()
    assert _serves(dst)
    st = to_np(dst.access_log_state())
    assert st[1] == len(otab) and st[2] == 0 and st[3] == otab.live()[1].min()
    _check_select(htl, dst, otab, 1, 3)
    _continue_stream(htl, orc, dst, otab, spec, range(5, 9))


def test_log_rebuilt_after_a_resize(htl, orc):
    spec = workloads.DynamicOnlineSpec(window=1 << 13, n=1 << 12, capacity_log2=15, dim=8)
    table = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, growable=True, access_log=True)
    otab = orc.Table(1 << spec.capacity_log2, spec.dim, orc.BF16)
    _continue_stream(htl, orc, table, otab, spec, range(4))
    table.resize(spec.capacity_log2 + 1)
    otab.resize(table.capacity)
    assert not _serves(table)
    table.rebuild_access_log()
    _continue_stream(htl, orc, table, otab, spec, range(4, 8))


def test_log_rebuild_refuses_a_wide_step_span_and_tables_without_a_log(htl, orc):
    table, otab, rng = _filled(htl, orc)
    ks = np.arange(50_000, 50_500, dtype=np.int64)
    table.find_or_insert(torch.from_numpy(ks).cuda(), step=70_000)     # ends the log (span)
    otab.find_or_insert(ks, step=70_000)
    with pytest.raises(htl.HTLError):
        table.rebuild_access_log()
    assert not _serves(table)
    _check_select(htl, table, otab, 1, 2)
    plain = htl.Table(10, 4, "bf16", last_seen=True)
    with pytest.raises(htl.HTLError):
        plain.rebuild_access_log()
    empty = htl.Table(12, 4, "bf16", last_seen=True, access_log=True)
    empty.rebuild_access_log()
    assert _serves(empty)
