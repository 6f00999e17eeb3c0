"""Full-size runs of the pooled, online and backward workloads, in the launch
shapes bench.py times, checked against the oracle value by value: every
pooled bag, every key's status, the live set with its last_seen stamps and
the eviction victims of every step.

Merged tables: 65,536 samples x 26 bags of Poisson(20) IDs (34.08M IDs), one
2^26-slot bf16 table of dim 128 warmed by an earlier batch.  Online: the
2^27-slot bf16 table of dim 64 over all 50 steps of the drifting stream,
the oracle table stepped beside it, once on a table whose eviction choice
scans last_seen and once on a table with the access log (the form bench.py
times), whose choice is served by the log at every step.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [True, False])
def test_merged_tables_full_size(htl, orc, fused):
    w = workloads.merged_tables()
    warm = workloads.merged_tables(seed=1)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    wk = torch.from_numpy(warm.keys).cuda()
    u0, _, n0 = htl.dedup_unique_inverse(wk)
    table.find_or_insert(u0, n_dev=n0)
    warm_u = to_np(u0)[:int(n0.item())]
    del wk, u0
    keys = torch.from_numpy(w.keys).cuda()
    offsets = torch.from_numpy(w.offsets).cuda()
    out, uniq, inv, nu, slots, status = htl.lookup(table, keys, offsets=offsets, out_dtype="bf16", fused=fused)
    U = int(nu.item())
    u = to_np(uniq)[:U]
    assert np.array_equal(np.sort(u), np.unique(w.keys))
    assert np.array_equal(u[to_np(inv)], w.keys)
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.BF16)
    assert np.all(otab.find_or_insert(warm_u) == orc.INSERTED)
    assert np.array_equal(to_np(status)[:U], otab.find_or_insert(u))
    got = to_np(out)
    del out
    want = otab.gather_pool(w.keys, w.offsets, orc.BF16)
    assert got.shape == want.shape and np.array_equal(got, want)


class _OnlineRun:
    """The online stream stepped on the GPU table and the oracle table side by
    side; advance(s_end) runs every step below s_end not yet run and checks,
    per step: each unique key's status, the live keys with their last_seen
    stamps, the victims and the erase statuses; the gathered rows in full
    every tenth step and on a fixed sample of 2^16 IDs at the others."""

    FULL_ROWS = (0, 10, 20, 30, 40, 49)

    def __init__(self, htl, orc, access_log):
        import concurrent.futures as cf
        self.htl, self.orc = htl, orc
        self.access_log = access_log
        self.spec = workloads.DynamicOnlineSpec()
        self.gen = workloads.DynamicOnlineStream(self.spec, self.spec.steps)
        # the host draws the key batches ahead on a few threads
        self.pool = cf.ThreadPoolExecutor(max_workers=4)
        self.batches = {s: self.pool.submit(self.gen.keys, s) for s in range(self.spec.steps)}
        self.table = htl.Table(self.spec.capacity_log2, self.spec.dim, "bf16", last_seen=True,
                               access_log=access_log)
        self.otab = orc.Table(1 << self.spec.capacity_log2, self.spec.dim, orc.BF16)
        self.sample = np.random.default_rng(17).integers(0, self.spec.n, 1 << 16)
        self.next = 0

    def step(self, s):
        htl, orc, spec = self.htl, self.orc, self.spec
        keys_np = self.batches.pop(s).result()
        keys = torch.from_numpy(keys_np).cuda()
        # even steps through the one-call forward, odd steps through the three calls
        out, uniq, inv, nu, slots, status = htl.lookup(self.table, keys, step=s, fused=(s % 2 == 0))
        U = int(nu.item())
        u = to_np(uniq)[:U]
        assert np.array_equal(u[to_np(inv)], keys_np), s          # also: u holds every key of the batch
        assert np.unique(u).size == U, s                           # ... once
        assert np.array_equal(to_np(status)[:U], self.otab.find_or_insert(u, step=s)), s
        if s in self.FULL_ROWS:
            got = to_np(out)
            assert np.array_equal(got, self.otab.gather(keys_np)), s
            del got
        else:
            idx = self.sample
            assert np.array_equal(to_np(out[torch.from_numpy(idx).cuda()]), self.otab.gather(keys_np[idx])), s
        del out
        k_all, ls_all, _, n_all = self.table.scan()
        L = int(n_all.item())
        lk, order = torch.sort(k_all[:L])                           # key order, on the device
        lls = ls_all[:L][order]
        ok, ols = self.otab.live()
        assert np.array_equal(to_np(lk), ok), s
        assert np.array_equal(to_np(lls).astype(np.uint32), ols), s
        del k_all, ls_all, lk, lls, order
        if self.access_log:
            # the log still vouches for every live key, so it serves the choice
            assert int(self.table.access_log_state()[0].item()) == 1, s
        victims, nv = self.table.lru_select(spec.evict_num, spec.evict_den)
        k = int(nv.item())
        want_v = self.otab.lru_victims(spec.evict_num, spec.evict_den)
        assert k == want_v.size, s
        assert np.array_equal(to_np(torch.sort(victims[:k])[0]), np.sort(want_v)), s
        est = to_np(self.table.erase(victims[:k]))
        assert np.all(est == htl.ERASED), s
        assert np.all(self.otab.erase(want_v) == orc.ERASED), s

    def advance(self, s_end):
        while self.next < s_end:
            self.step(self.next)
            self.next += 1

    def close(self):
        self.pool.shutdown(wait=True, cancel_futures=True)


@pytest.fixture(scope="module", params=[False, True], ids=["scan", "access_log"])
def online_run(htl, orc, request):
    run = _OnlineRun(htl, orc, request.param)
    yield run
    run.close()
    del run.table
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("s_end", [10, 20, 30, 40, 50])
def test_online_full_size_steps(online_run, s_end):
    # all 50 steps of the online stream in five parts (each part runs the
    # steps the parts before it left, so a part run alone checks from step 0)
    online_run.advance(s_end)


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
