"""GPU parity of the one-call forward lookup (emb_lookup) against the oracle
and against the three calls it replaces.

emb_lookup runs the dedup, find-or-insert and the gather (or bag pooling) in
one call, composing each ID's slot after find-or-insert instead of reading
slots[inverse[i]] in the gather.  Its outputs must be what the three calls
give: the same unique set and inverse mapping, every key's status as the
oracle table reports it, and every gathered row or pooled bag bit-exact --
for each form of the dedup's second stage (one tile, hash bins, device set),
for fixed and growable tables, and for bf16 rows widened to fp32.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _check_forward(htl, orc, table, otab, keys_np, res, offsets_np=None, out_dtype=None, step=0):
    out, uniq, inv, nu, slots, status = res
    U = int(nu.item())
    ref_u, _ = orc.dedup(keys_np)
    u = to_np(uniq)[:U]
    assert U == ref_u.size and np.array_equal(np.sort(u), ref_u)
    if keys_np.size:
        assert np.array_equal(u[to_np(inv)], keys_np)
    ref_st = otab.find_or_insert(u, step=step)
    assert np.array_equal(to_np(status)[:U], ref_st)
    if offsets_np is None:
        want = otab.gather(keys_np)
        got = to_np(out)
        if table.dtype == htl.BF16 and out_dtype == "f32":
            want = orc.bf16_bits_to_f32(want)
        assert np.array_equal(got, want)
    elif table.dtype == htl.BF16:
        # bf16 rows: every fp32 partial sum is exact, so the sums are bit-exact
        od = orc.BF16 if out_dtype == "bf16" else orc.F32
        assert np.array_equal(to_np(out), otab.gather_pool(keys_np, offsets_np, od))
    else:
        _check_f32_pool(orc, otab, keys_np, offsets_np, to_np(out))


def _check_f32_pool(orc, otab, keys_np, offsets_np, got):
    # fp32 rows summed in fp32 in an unspecified order: within 1e-5 of the
    # bag's sum of |row| (the summation-error scale), against fp64 sums
    ref = otab.gather_pool(keys_np, offsets_np, orc.F32).astype(np.float64)
    rows = np.abs(otab.gather(keys_np).astype(np.float64))
    nz = np.diff(offsets_np) > 0
    absum = np.zeros_like(ref)
    absum[nz] = np.add.reduceat(rows, offsets_np[:-1][nz], axis=0)
    got = got.astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-5 * absum)
    assert not got[~nz].any()


@pytest.mark.parametrize("n", [0, 1, 2047, 2048, 2049, 6144 + 5, 100_003, 1 << 20])
def test_fused_lookup_sizes(htl, orc, n):
    w = workloads.tiny(seed=n, n=max(n, 1))
    keys_np = w.keys[:n]
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.F32)
    for step in range(2):          # the second pass finds every key
        res = htl.lookup(table, torch.from_numpy(keys_np).cuda(), step=step, fused=True)
        _check_forward(htl, orc, table, otab, keys_np, res, step=step)


@pytest.mark.parametrize("path", ["bins", "set"])
def test_fused_lookup_matches_three_calls(htl, orc, monkeypatch, path):
    # the large-table shape at 1/8 size, through each stage-2 form
    if path == "set":
        monkeypatch.setenv("HTL_DEDUP_PATH", "set")
    w = workloads.single_large_table(n=1 << 19, capacity_log2=21, prefill_count=1 << 20)
    keys = torch.from_numpy(w.keys).cuda()
    pre = torch.from_numpy(w.prefill).cuda()
    outs = []
    for fused in (True, False):
        t = htl.Table(w.capacity_log2, w.dim, w.dtype)
        t.find_or_insert(pre)
        outs.append(htl.lookup(t, keys, fused=fused))
    a, b = outs
    Ua, Ub = int(a[3].item()), int(b[3].item())
    assert Ua == Ub
    ua, ub = to_np(a[1])[:Ua], to_np(b[1])[:Ub]
    assert np.array_equal(np.sort(ua), np.sort(ub))
    assert np.array_equal(ua[to_np(a[2])], w.keys) and np.array_equal(ub[to_np(b[2])], w.keys)
    sa = dict(zip(ua.tolist(), to_np(a[5])[:Ua].tolist()))
    sb = dict(zip(ub.tolist(), to_np(b[5])[:Ub].tolist()))
    assert sa == sb
    assert torch.equal(a[0], b[0])
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.F32)
    otab.find_or_insert(w.prefill)
    st = otab.find_or_insert(ua)
    assert np.array_equal(to_np(a[5])[:Ua], st)
    assert np.array_equal(to_np(a[0]), otab.gather(w.keys))


@pytest.mark.parametrize("path", ["bins", "set"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_fused_pooled_lookup(htl, orc, monkeypatch, path, out_dtype):
    if path == "set":
        monkeypatch.setenv("HTL_DEDUP_PATH", "set")
    m = workloads.merged_tables(batch=2048, capacity_log2=20)
    table = htl.Table(m.capacity_log2, m.dim, m.dtype)
    otab = orc.Table(1 << m.capacity_log2, m.dim, orc.BF16)
    offsets = torch.from_numpy(m.offsets).cuda()
    keys = torch.from_numpy(m.keys).cuda()
    for step in range(2):
        res = htl.lookup(table, keys, step=step, offsets=offsets, out_dtype=out_dtype, fused=True)
        _check_forward(htl, orc, table, otab, m.keys, res, offsets_np=m.offsets, out_dtype=out_dtype, step=step)


def test_fused_lookup_widen_and_empty_bags(htl, orc):
    # bf16 rows widened to fp32 per ID, then bags with empty ones at both ends
    rng = np.random.default_rng(5)
    keys_np = rng.integers(0, 5000, 9000).astype(np.int64) * 31 + 7
    table = htl.Table(16, 24, "bf16")
    otab = orc.Table(1 << 16, 24, orc.BF16)
    res = htl.lookup(table, torch.from_numpy(keys_np).cuda(), out_dtype="f32", fused=True)
    _check_forward(htl, orc, table, otab, keys_np, res, out_dtype="f32")
    lens = rng.integers(0, 7, 2000)
    lens[:3] = 0
    lens[-3:] = 0
    offsets_np = np.zeros(lens.size + 1, dtype=np.int32)
    np.cumsum(lens, out=offsets_np[1:])
    k2 = rng.integers(0, 3000, int(offsets_np[-1])).astype(np.int64) * 17 + 1
    res = htl.lookup(table, torch.from_numpy(k2).cuda(), step=1, offsets=torch.from_numpy(offsets_np).cuda(),
                     out_dtype="bf16", fused=True)
    _check_forward(htl, orc, table, otab, k2, res, offsets_np=offsets_np, out_dtype="bf16", step=1)


def test_fused_lookup_growable_table(htl, orc):
    # row handles instead of slots: the composed per-ID handles feed the gather
    w = workloads.tiny(seed=9, n=150_000)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype, growable=True)
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.F32)
    for step in range(2):
        res = htl.lookup(table, torch.from_numpy(w.keys).cuda(), step=step, fused=True)
        _check_forward(htl, orc, table, otab, w.keys, res, step=step)


def test_fused_lookup_reserved_keys(htl, orc):
    # the table's marker values come back RESERVED with a zero row, as in the
    # three calls
    keys_np = np.array([5, -1, 7, -2, 5, 9] * 700, dtype=np.int64)
    table = htl.Table(12, 8, "f32")
    out, uniq, inv, nu, slots, status = htl.lookup(table, torch.from_numpy(keys_np).cuda(), fused=True)
    U = int(nu.item())
    u, st = to_np(uniq)[:U], to_np(status)[:U]
    by_key = dict(zip(u.tolist(), st.tolist()))
    assert by_key == {5: htl.INSERTED, 7: htl.INSERTED, 9: htl.INSERTED, -1: htl.RESERVED, -2: htl.RESERVED}
    o = to_np(out)
    assert np.all(o[keys_np < 0] == 0)
    assert np.array_equal(o[keys_np == 5], orc.init_rows(keys_np[keys_np == 5], 8, orc.F32))


@pytest.mark.parametrize("kind", ["f32", "bf16", "adam", "dim6", "growable"])
@pytest.mark.parametrize("pooled", [False, True])
def test_fused_lookup_leaves_initial_rows_in_the_table(htl, orc, kind, pooled):
    # after the call, every unique key's row in the table (read back at the
    # slot the call returned) is the oracle's row, for tables of each kind
    dtype = "bf16" if kind == "bf16" else "f32"
    dim = 6 if kind == "dim6" else 32
    table = htl.Table(17, dim, dtype, adam=(kind == "adam"), growable=(kind == "growable"))
    otab = orc.Table(1 << 17, dim, orc.BF16 if dtype == "bf16" else orc.F32)
    rng = np.random.default_rng(3)
    pre = rng.integers(0, 1 << 40, 20_000).astype(np.int64)
    table.find_or_insert(torch.from_numpy(np.unique(pre)).cuda())
    otab.find_or_insert(np.unique(pre))
    keys_np = np.concatenate([pre[:10_000], rng.integers(0, 1 << 40, 60_000)]).astype(np.int64)
    keys_np = keys_np[rng.permutation(keys_np.size)]
    offsets_np = None
    offsets = None
    if pooled:
        lens = rng.integers(0, 9, 12_000)
        offsets_np = np.zeros(lens.size + 1, dtype=np.int32)
        np.cumsum(lens, out=offsets_np[1:])
        keys_np = keys_np[:int(offsets_np[-1])]
        offsets = torch.from_numpy(offsets_np).cuda()
    res = htl.lookup(table, torch.from_numpy(keys_np).cuda(), step=1, offsets=offsets, fused=True)
    _check_forward(htl, orc, table, otab, keys_np, res, offsets_np=offsets_np,
                   out_dtype=dtype if pooled else None, step=1)
    _, uniq, _, nu, slots, _ = res
    U = int(nu.item())
    rows = htl.gather(table, slots[:U].contiguous())
    assert np.array_equal(to_np(rows), otab.gather(to_np(uniq)[:U]))
