"""Full-size runs of the pooled and online workloads, in the launch shapes
bench.py times, checked on what the oracle computes one by one (closed-form
rows of sampled keys, brute-force sums of sampled bags) and on properties
that hold at any size (unique set, inverse, LRU order, erase statuses).

Merged tables: 65,536 samples x 26 bags of Poisson(20) IDs (34.08M IDs), one
2^26-slot bf16 table of dim 128 warmed by an earlier batch.  Online: the
2^27-slot bf16 table of dim 64 over the first steps of the drifting stream.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_merged_tables_full_size(htl, orc):
    w = workloads.merged_tables()
    warm = workloads.merged_tables(seed=1)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    wk = torch.from_numpy(warm.keys).cuda()
    u0, _, n0 = htl.dedup_unique_inverse(wk)
    table.find_or_insert(u0, n_dev=n0)
    del wk, u0
    keys = torch.from_numpy(w.keys).cuda()
    offsets = torch.from_numpy(w.offsets).cuda()
    out, uniq, inv, nu, slots, status = htl.lookup(table, keys, offsets=offsets, out_dtype="bf16")
    U = int(nu.item())
    u = to_np(uniq)[:U]
    assert np.array_equal(np.sort(u), np.unique(w.keys))
    sample = np.random.default_rng(3).integers(0, w.keys.size, 1 << 16)
    assert np.array_equal(u[to_np(inv)[sample]], w.keys[sample])
    st = to_np(status)[:U]
    assert np.array_equal(st == htl.FOUND, np.isin(u, warm.keys))
    # sampled bags: brute-force fp64 sums of closed-form bf16 rows, rounded
    # to bf16 (exact in fp32 in any order, so bit-equal)
    rng = np.random.default_rng(4)
    bags = np.concatenate([rng.integers(0, w.nbags, 3000), [0, w.nbags - 1]])
    got = to_np(out[torch.from_numpy(bags).cuda()])
    for b, row in zip(bags, got):
        ks = w.keys[w.offsets[b]:w.offsets[b + 1]]
        if ks.size == 0:
            assert np.all(row == 0)
            continue
        rows = orc.bf16_bits_to_f32(orc.init_rows(ks, w.dim, orc.BF16)).astype(np.float64)
        s = rows.sum(axis=0).astype(np.float32)
        want = (s.view(np.uint32) + 0x7FFF + ((s.view(np.uint32) >> 16) & 1)) >> 16
        assert np.array_equal(row, want.astype(np.uint16)), b


def test_online_full_size_steps(htl, orc):
    spec = workloads.DynamicOnlineSpec()
    steps = 3
    gen = workloads.DynamicOnlineStream(spec, steps)
    table = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True)
    live_before = 0
    for s in range(steps):
        keys_np = gen.keys(s)
        keys = torch.from_numpy(keys_np).cuda()
        out, uniq, inv, nu, slots, status = htl.lookup(table, keys, step=s)
        U = int(nu.item())
        u = to_np(uniq)[:U]
        st = to_np(status)[:U]
        assert np.array_equal(np.sort(u), np.unique(keys_np))
        ins = st == htl.INSERTED
        assert np.all((st == htl.FOUND) | ins)
        idx = np.random.default_rng(s).integers(0, keys_np.size, 2048)
        assert np.array_equal(to_np(out[torch.from_numpy(idx).cuda()]),
                              orc.init_rows(keys_np[idx], spec.dim, orc.BF16))
        k_all, ls_all, _, n_all = table.scan()
        L = int(n_all.item())
        assert L == live_before + int(ins.sum())
        victims, nv = table.lru_select(spec.evict_num, spec.evict_den)
        k = int(nv.item())
        assert k == L * spec.evict_num // spec.evict_den
        vk = to_np(victims)[:k]
        lk, lls = to_np(k_all)[:L], to_np(ls_all)[:L].astype(np.uint32)
        order = np.lexsort((lk, lls))                      # by (last_seen, key)
        assert np.array_equal(np.sort(vk), np.sort(lk[order[:k]]))
        est = to_np(table.erase(victims[:k]))
        assert np.all(est == htl.ERASED)
        live_before = L - k


def test_backward_fused_full_size_matches_two_calls(htl):
    """2^23 IDs Zipf(1.2), dim 128, at full size: the fused segment-sum + Adam
    gives bit-for-bit the rows, m and v of segment-sum then Adam, with
    gradients that are multiples of 2^-6 in [-1/8, 1/8] (every segment sum,
    up to the hottest key's 1.5M rows, is exact in fp32, so the order of
    summation cannot matter)."""
    w = workloads.backward(with_grad=False)
    n, dim = w.keys.size, w.dim
    keys = torch.from_numpy(w.keys).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    grad = torch.randint(-8, 9, (n, dim), generator=gen, device="cuda").to(torch.float32) * 2.0 ** -6
    uniq, inv, nu = htl.dedup_unique_inverse(keys, ordered=True)
    U = int(nu.item())
    res = []
    for fused in (True, False):
        t = htl.Table(w.capacity_log2, dim, "f32", adam=True)
        slots, _ = t.find_or_insert(uniq, n_dev=nu)
        if fused:
            htl.segment_sum_adam(t, slots, grad, inv, nu, n)
        else:
            g = htl.segment_sum(grad, inv, nu, u_max=n)
            htl.rowwise_adam(t, slots, g, nu, 1e-3, 0.9, 0.999, 1e-8, 1)
            del g
        sl = slots[:U].long()
        res.append([htl.table_tensor(t, name)[sl].cpu() for name in ("rows", "adam_m", "adam_v")])
        del t
        torch.cuda.empty_cache()
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("path", ["bins", "bins_in_device_memory", "set"])
def test_large_table_batch_dedup_paths(htl, orc, monkeypatch, path):
    # the large-table batch (2^22 Zipf IDs) through each form of the second
    # dedup stage: LDS bins (the default), every bin redone in device memory,
    # and the device-wide set -- the same unique set and a correct inverse
    if path == "bins_in_device_memory":
        monkeypatch.setenv("HTL_DEDUP_BIN_MAX", "0")
    if path == "set":
        monkeypatch.setenv("HTL_DEDUP_PATH", "set")
    w = workloads.single_large_table()
    keys = torch.from_numpy(w.keys).cuda()
    uniq, inv, nu = htl.dedup_unique_inverse(keys)
    U = int(nu.item())
    u = to_np(uniq)[:U]
    ref = np.unique(w.keys)
    assert U == ref.size and np.array_equal(np.sort(u), ref)
    assert np.array_equal(u[to_np(inv)], w.keys)


@pytest.mark.parametrize("n", [1 << 23, (1 << 23) + 1])
def test_dedup_at_the_partitioned_limit(htl, n):
    # 2^23 keys is the largest batch the hash-binned second stage takes
    # (all distinct: ~2048 distinct keys per bin, the most its LDS sets see
    # for random keys); one key more goes to the device set
    rng = np.random.default_rng(n)
    distinct = rng.choice(1 << 40, size=n, replace=False).astype(np.int64) * 7 + 3
    for keys in (distinct, distinct[rng.integers(0, n // 3, n)]):
        uniq, inv, nu = htl.dedup_unique_inverse(torch.from_numpy(keys).cuda())
        U = int(nu.item())
        u = to_np(uniq)[:U]
        ref = np.unique(keys)
        assert U == ref.size and np.array_equal(np.sort(u), ref)
        assert np.array_equal(u[to_np(inv)], keys)
