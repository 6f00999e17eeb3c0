"""GPU parity of the forward path against the CPU oracle.

dedup_unique_inverse, ht_find_or_insert, emb_gather_pool are called through
the C ABI (via the ctypes binding) and compared with the oracle on the same
seeded inputs.  Slot placement and unique order depend on GPU scheduling, so
what is compared is what is unique: the set of unique keys, the map
ID -> key through the inverse, the status of every key, and every gathered or
pooled row -- all bit-exact.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _dedup_check(htl, orc, keys_np, ordered=False):
    keys = torch.from_numpy(keys_np).cuda()
    uniq, inv, nu = htl.dedup_unique_inverse(keys, ordered=ordered)
    U = int(nu.item())
    u = to_np(uniq)[:U]
    i = to_np(inv)
    ref_u, ref_inv = orc.dedup(keys_np)
    assert U == ref_u.size
    assert np.array_equal(np.sort(u), ref_u)               # same set, no duplicates
    if keys_np.size:
        assert i.min() >= 0 and i.max() < U
        assert np.array_equal(u[i], keys_np)               # inverse maps back
        # canonical inverse: rank of each ID's key in the sorted unique list
        assert np.array_equal(np.searchsorted(ref_u, u[i]).astype(np.int32), ref_inv)
    return u, i, U


@pytest.mark.parametrize("ordered", [False, True])
@pytest.mark.parametrize("n", [0, 1, 2, 2047, 2048, 2049, 6144 + 5, 65536, 100_003])
def test_dedup_sizes(htl, orc, n, ordered):
    rng = np.random.default_rng(n)
    keys = rng.integers(0, max(4, n // 3), n).astype(np.int64) * 977 - 5
    u, _, _ = _dedup_check(htl, orc, keys, ordered)
    if ordered and n:
        _, first = np.unique(keys, return_index=True)
        assert np.array_equal(u, keys[np.sort(first)])


@pytest.mark.parametrize("seed", [0, 1])
def test_dedup_first_occurrence_order(htl, orc, seed):
    # unique[] lists keys in order of first occurrence, so the whole output is
    # a function of the input alone; checked against numpy's first indices.
    w = workloads.tiny(seed=seed, n=300_000 + seed * 777)
    u, i, U = _dedup_check(htl, orc, w.keys, ordered=True)
    _, first = np.unique(w.keys, return_index=True)
    assert np.array_equal(u, w.keys[np.sort(first)])
    u2, i2, _ = _dedup_check(htl, orc, w.keys, ordered=True)
    assert np.array_equal(u, u2) and np.array_equal(i, i2)


@pytest.mark.parametrize("ordered", [False, True])
def test_dedup_special_values(htl, orc, ordered):
    i64 = np.iinfo(np.int64)
    base = np.array([-1, -2, i64.min, i64.max, 0, 1, -1, i64.min], dtype=np.int64)
    rng = np.random.default_rng(1)
    keys = np.concatenate([base, rng.choice(base, 5000), rng.integers(-50, 50, 5000)])
    rng.shuffle(keys)
    _dedup_check(htl, orc, keys, ordered)
    _dedup_check(htl, orc, base, ordered)                               # one-tile batches (single launch)
    _dedup_check(htl, orc, rng.choice(base, 2048), ordered)
    _dedup_check(htl, orc, np.full(70000, -1, np.int64), ordered)     # only the out-of-band key
    _dedup_check(htl, orc, np.full(70000, 12345, np.int64), ordered)  # all equal
    _dedup_check(htl, orc, rng.permutation(150000).astype(np.int64), ordered)   # all distinct


def _dedup_cases(rng):
    i64 = np.iinfo(np.int64)
    base = np.array([-1, -2, i64.min, i64.max, 0, 1], dtype=np.int64)
    return [
        rng.integers(0, 30_000, 100_003).astype(np.int64) * 977 - 5,
        np.concatenate([rng.choice(base, 9000), rng.integers(-300, 300, 9000)]),
        rng.permutation(150_000).astype(np.int64),                      # all distinct
        np.full(70_000, -1, np.int64),                                  # only the out-of-band key
    ]


@pytest.mark.parametrize("bin_max", ["0", "3", "200"])
def test_dedup_bins_redone_in_device_memory(htl, orc, monkeypatch, bin_max):
    # Bins whose distinct keys outgrow the LDS set are redone in device
    # memory; lowering the LDS limit sends some or all bins that way.
    monkeypatch.setenv("HTL_DEDUP_BIN_MAX", bin_max)
    for keys in _dedup_cases(np.random.default_rng(int(bin_max))):
        _dedup_check(htl, orc, keys)


def test_dedup_set_path(htl, orc, monkeypatch):
    # The device-set stage 2 (the ordered mode's, and very large batches')
    # also serves the unordered mode when asked.
    monkeypatch.setenv("HTL_DEDUP_PATH", "set")
    for keys in _dedup_cases(np.random.default_rng(7)):
        _dedup_check(htl, orc, keys)


def test_dedup_tiny_workload(htl, orc):
    w = workloads.tiny()
    _, _, U = _dedup_check(htl, orc, w.keys)
    assert U == np.unique(w.keys).size


def _lookup_parity(htl, orc, keys_np, capacity_log2, dim, dtype, prefill=None, step=0, seed=0):
    """Run dedup -> find_or_insert -> gather on GPU and oracle; compare all outputs."""
    odt = orc.F32 if dtype == "f32" else orc.BF16
    table = htl.Table(capacity_log2, dim, dtype, init_seed=seed)
    otab = orc.Table(1 << capacity_log2, dim, odt, seed=seed)
    if prefill is not None and prefill.size:
        pf = torch.from_numpy(prefill).cuda()
        _, st = table.find_or_insert(pf)
        assert np.all(to_np(st) == htl.INSERTED)
        otab.find_or_insert(prefill)
    keys = torch.from_numpy(keys_np).cuda()
    out, uniq, inv, nu, slots, status = htl.lookup(table, keys, step=step)
    U = int(nu.item())
    u = to_np(uniq)[:U]
    st = to_np(status)[:U]
    sl = to_np(slots)[:U]
    ref_u, _ = orc.dedup(keys_np)
    assert np.array_equal(np.sort(u), ref_u)
    ref_st = otab.find_or_insert(u, step=step)       # same call order: statuses are order-free here
    assert np.array_equal(st, ref_st)
    assert np.all(sl[st <= 1] >= 0) and np.unique(sl[st <= 1]).size == int((st <= 1).sum())
    got = to_np(out)
    ref = otab.gather(keys_np)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)
    return table, otab, u, st, sl


def test_tiny_insert_then_find(htl, orc):
    w = workloads.tiny()
    table, otab, u, st, sl = _lookup_parity(htl, orc, w.keys, w.capacity_log2, w.dim, w.dtype)
    assert np.all(st == htl.INSERTED)
    # the same batch again: every key FOUND, same slots
    keys = torch.from_numpy(w.keys).cuda()
    out, uniq, inv, nu, slots, status = htl.lookup(table, keys, step=1)
    U = int(nu.item())
    u2, st2, sl2 = to_np(uniq)[:U], to_np(status)[:U], to_np(slots)[:U]
    assert np.all(st2 == htl.FOUND)
    assert dict(zip(u.tolist(), sl.tolist())) == dict(zip(u2.tolist(), sl2.tolist()))
    assert np.array_equal(to_np(out), otab.gather(w.keys))


@pytest.mark.parametrize("dim,dtype", [(16, "f32"), (64, "f32"), (128, "bf16"), (64, "bf16"),
                                       (3, "f32"), (5, "bf16"), (24, "bf16"), (200, "f32")])
def test_row_shapes(htl, orc, dim, dtype):
    rng = np.random.default_rng(dim)
    keys = rng.integers(0, 5000, 20000).astype(np.int64) << np.int64(20)
    _lookup_parity(htl, orc, keys, 14, dim, dtype, seed=dim)


def test_single_large_table_shape_small(htl, orc):
    # the large-table workload's shape at 1/64 scale: half the slots pre-filled
    w = workloads.single_large_table(n=1 << 16, capacity_log2=18, prefill_count=1 << 17)
    _, _, u, st, _ = _lookup_parity(htl, orc, w.keys, w.capacity_log2, w.dim, w.dtype, prefill=w.prefill)
    pre = np.isin(u, w.prefill)
    assert np.array_equal(st == htl.FOUND, pre)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6])
def test_fill_to_full(htl, orc, k):
    M = 1 << k
    table = htl.Table(k, 4, "f32")
    keys = torch.arange(M, dtype=torch.int64, device="cuda") * 1000 + 3
    slots, st = table.find_or_insert(keys)
    assert np.all(to_np(st) == htl.INSERTED)
    assert sorted(to_np(slots).tolist()) == list(range(M))   # every slot reachable (Theorem 1)
    _, st = table.find_or_insert(torch.tensor([999_999], dtype=torch.int64, device="cuda"))
    assert to_np(st).tolist() == [htl.FULL]
    _, st = table.find_or_insert(keys)
    assert np.all(to_np(st) == htl.FOUND)
    # more new keys than free slots in one call: exactly `free` of them get in
    er = table.erase(keys[:3] if M >= 3 else keys[:1])
    freed = int((to_np(er) == htl.ERASED).sum())
    new = torch.arange(5, dtype=torch.int64, device="cuda") + 10**9
    _, st = table.find_or_insert(new)
    st = to_np(st)
    assert int((st == htl.INSERTED).sum()) == freed and int((st == htl.FULL).sum()) == 5 - freed


def test_reserved_keys(htl, orc):
    table = htl.Table(8, 4, "f32")
    keys = torch.tensor([-1, 7, -2, 8], dtype=torch.int64, device="cuda")
    slots, st = table.find_or_insert(keys)
    assert to_np(st).tolist() == [htl.RESERVED, htl.INSERTED, htl.RESERVED, htl.INSERTED]
    assert to_np(slots)[[0, 2]].tolist() == [-1, -1]
    assert to_np(table.erase(keys)).tolist() == [htl.NOT_FOUND, htl.ERASED, htl.NOT_FOUND, htl.ERASED]


def _oracle_in_gpu_order(otab, keys, st_gpu, step, full_code):
    """When a call runs out of free slots, which new keys get FULL depends on
    arrival order.  Replay the oracle with the keys the GPU admitted first:
    the GPU's statuses are valid iff this order reproduces them exactly."""
    order = np.argsort(st_gpu == full_code, kind="stable")
    ref = np.empty_like(st_gpu)
    ref[order] = otab.find_or_insert(keys[order], step=step)
    return ref


def test_erase_tombstones_and_reinsert(htl, orc):
    # 6000 possible keys churn through 4096 slots: tombstones pile up and the
    # last rounds run the table full
    rng = np.random.default_rng(5)
    table = htl.Table(12, 8, "f32")
    otab = orc.Table(1 << 12, 8)
    saw_full = False
    for rnd in range(8):
        ins = np.unique(rng.integers(0, 6000, 2500)).astype(np.int64)
        rng.shuffle(ins)
        _, st = table.find_or_insert(torch.from_numpy(ins).cuda(), step=rnd)
        st = to_np(st)
        saw_full |= bool((st == htl.FULL).any())
        assert np.array_equal(st, _oracle_in_gpu_order(otab, ins, st, rnd, htl.FULL))
        er = np.unique(rng.integers(0, 6000, 1500)).astype(np.int64)
        st = table.erase(torch.from_numpy(er).cuda())
        assert np.array_equal(to_np(st), otab.erase(er))
        keys, ls, slots, n = table.scan()
        L = int(n.item())
        assert L == len(otab)
        assert np.array_equal(np.sort(to_np(keys)[:L]), otab.live()[0])
    assert saw_full
    # rows of live keys are still their closed-form rows after tombstone reuse
    lk = otab.live()[0]
    slots, st = table.find_or_insert(torch.from_numpy(lk).cuda())
    assert np.all(to_np(st) == htl.FOUND)
    got = to_np(htl.gather(table, slots))
    assert np.array_equal(got, otab.gather(lk))


def test_duplicate_erase_reports_once(htl, orc):
    table = htl.Table(10, 4, "f32")
    table.find_or_insert(torch.tensor([5, 6], dtype=torch.int64, device="cuda"))
    st = to_np(table.erase(torch.tensor([5] * 100 + [6], dtype=torch.int64, device="cuda")))
    assert int((st[:100] == htl.ERASED).sum()) == 1 and st[100] == htl.ERASED


@pytest.mark.parametrize("fused", [True, False])
def test_repeatable(htl, orc, fused):
    # the same batch into ten fresh tables: the unique set, every key's status
    # and every row must come out the same each time (a lost or doubled CAS
    # claim would change them)
    w = workloads.tiny(seed=3, n=200_000)
    keys = torch.from_numpy(w.keys).cuda()
    first = None
    for _ in range(10):
        table = htl.Table(w.capacity_log2, w.dim, w.dtype)
        out, uniq, inv, nu, slots, status = htl.lookup(table, keys, fused=fused)
        U = int(nu.item())
        u, st = to_np(uniq)[:U], to_np(status)[:U]
        order = np.argsort(u)
        got = (u[order], st[order], to_np(out))
        assert np.all(got[1] == htl.INSERTED)
        assert np.unique(to_np(slots)[:U]).size == U              # one slot per key
        if first is None:
            first = got
        else:
            for a, b in zip(got, first):
                assert np.array_equal(a, b)


def test_pool_merged_tables_small(htl, orc):
    w = workloads.merged_tables(batch=1024, capacity_log2=20)
    for out_dtype, odt in (("bf16", orc.BF16), ("f32", orc.F32)):
        table = htl.Table(w.capacity_log2, w.dim, w.dtype)
        otab = orc.Table(1 << w.capacity_log2, w.dim, orc.BF16)
        keys = torch.from_numpy(w.keys).cuda()
        offs = torch.from_numpy(w.offsets).cuda()
        out, uniq, inv, nu, slots, status = htl.lookup(table, keys, offsets=offs, out_dtype=out_dtype)
        U = int(nu.item())
        otab.find_or_insert(to_np(uniq)[:U])
        ref = otab.gather_pool(w.keys, w.offsets, odt)
        assert np.array_equal(to_np(out), ref)


@pytest.mark.parametrize("dim,dtype", [(64, "bf16"), (16, "f32"), (512, "bf16"), (6, "bf16")])
def test_pool_offsets_that_break_the_rules(htl, orc, dim, dtype):
    # emb_gather_pool's contract for offsets outside the CSR rules: every bag
    # is clamped to [0, n) on its own, and a bag whose clamped start is not
    # below its clamped end sums nothing.  Offsets below 0, above n and
    # decreasing pairs, through the team-per-bag (dim 64, 16), wave-per-bag
    # (dim 512) and element-wise (dim 6) kernels; rows from the oracle.
    rng = np.random.default_rng(100 + dim)
    n, nb = 5000, 600
    keys = rng.integers(0, 700, n).astype(np.int64)
    offsets = np.sort(rng.integers(0, n + 1, nb + 1)).astype(np.int64)
    offsets[rng.choice(nb + 1, 40, replace=False)] = rng.integers(-50, 0, 40)
    offsets[rng.choice(nb + 1, 40, replace=False)] = rng.integers(n + 1, n + 100, 40)
    for s in rng.choice(nb, 40, replace=False):
        offsets[s], offsets[s + 1] = offsets[s + 1], offsets[s]
    beg, end = np.clip(offsets[:-1], 0, n), np.clip(offsets[1:], 0, n)
    assert (beg > end).sum() > 10 and (offsets < 0).any() and (offsets > n).any()
    uk, inv = np.unique(keys, return_inverse=True)
    table = htl.Table(12, dim, dtype)
    slots, st = table.find_or_insert(torch.from_numpy(uk).cuda())
    assert (to_np(st) == htl.INSERTED).all()
    got = to_np(htl.gather_pool(table, slots, torch.from_numpy(inv.astype(np.int32)).cuda(),
                                torch.from_numpy(offsets.astype(np.int32)).cuda(), out_dtype="f32"))
    otab = orc.Table(1 << 12, dim, orc.F32 if dtype == "f32" else orc.BF16)
    otab.find_or_insert(uk)
    rows = otab.gather(keys)
    rows = (orc.bf16_bits_to_f32(rows) if dtype == "bf16" else rows).astype(np.float64)
    want, bound = np.zeros((nb, dim)), np.zeros((nb, dim))
    for b in range(nb):
        if beg[b] < end[b]:
            want[b] = rows[beg[b]:end[b]].sum(axis=0)
            # recursive fp32 summation of L terms: |error| <= (L - 1) u sum|x|
            bound[b] = (end[b] - beg[b]) * 2.0**-24 * np.abs(rows[beg[b]:end[b]]).sum(axis=0)
    if dtype == "bf16":
        assert np.array_equal(got.astype(np.float64), want)   # sums of bf16 rows are exact in fp32
    else:
        assert (np.abs(got.astype(np.float64) - want) <= bound).all()
        assert np.array_equal(got[beg >= end], np.zeros(((beg >= end).sum(), dim), np.float32))
    table.close()


@pytest.mark.parametrize("dim,dtype", [(16, "f32"), (64, "bf16"), (6, "bf16"), (7, "f32"), (512, "bf16")])
def test_pool_shapes_and_empty_bags(htl, orc, dim, dtype):
    rng = np.random.default_rng(dim)
    lens = rng.poisson(3, 3000)
    lens[::7] = 0
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    keys = rng.integers(0, 800, offsets[-1]).astype(np.int64)
    odt = orc.F32 if dtype == "f32" else orc.BF16
    table = htl.Table(12, dim, dtype)
    otab = orc.Table(1 << 12, dim, odt)
    out, uniq, inv, nu, slots, status = htl.lookup(table, torch.from_numpy(keys).cuda(),
                                                   offsets=torch.from_numpy(offsets).cuda(), out_dtype="f32")
    otab.find_or_insert(np.unique(keys))
    ref = otab.gather_pool(keys, offsets, orc.F32)
    got = to_np(out)
    if dtype == "bf16":
        assert np.array_equal(got, ref)                 # exact sums
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-7)
    assert not got[lens == 0].any()


def test_widening_gather(htl, orc):
    rng = np.random.default_rng(9)
    keys = rng.integers(0, 3000, 9000).astype(np.int64)
    table = htl.Table(13, 64, "bf16")
    out, uniq, inv, nu, slots, status = htl.lookup(table, torch.from_numpy(keys).cuda(), out_dtype="f32")
    otab = orc.Table(1 << 13, 64, orc.BF16)
    otab.find_or_insert(np.unique(keys))
    ref = orc.bf16_bits_to_f32(otab.gather(keys))
    assert np.array_equal(to_np(out), ref)


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("fused", [True, False])
def test_single_large_table_full_size(htl, orc, fused):
    """The 2^22-ID / 2^24-slot workload at full size, in the launch shapes
    bench.py times (the one-call forward, and the three calls), against the
    oracle table pre-filled with the same 2^23 keys: the unique set, every
    ID's inverse, every unique key's status, and all 4,194,304 gathered rows
    bit for bit."""
    w = workloads.single_large_table()
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    _, st = table.find_or_insert(torch.from_numpy(w.prefill).cuda())
    assert np.all(to_np(st) == htl.INSERTED)
    keys = torch.from_numpy(w.keys).cuda()
    out, uniq, inv, nu, slots, status = htl.lookup(table, keys, fused=fused)
    U = int(nu.item())
    u = to_np(uniq)[:U]
    ref_u = np.unique(w.keys)
    assert np.array_equal(np.sort(u), ref_u)
    assert np.array_equal(u[to_np(inv)], w.keys)
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.F32)
    assert np.all(otab.find_or_insert(w.prefill) == orc.INSERTED)
    assert np.array_equal(to_np(status)[:U], otab.find_or_insert(u))
    got = to_np(out)
    del out
    want = otab.gather(w.keys)
    assert got.shape == want.shape and np.array_equal(got, want)


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (1 << 24) + 16])
def test_copy_probe(htl, nbytes):
    # the bandwidth reference kernel copies exactly
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    htl.copy_probe(src, dst)
    assert torch.equal(src, dst)
