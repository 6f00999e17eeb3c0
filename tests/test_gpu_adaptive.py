"""GPU parity of the dedup's stage-2 forms and of the adaptive choice
between them (dedup_unique_inverse_adaptive), against the oracle.

Every form -- one tile, two-stage hash bins, hash bins without stage 1, the
device-wide set -- must give the oracle's unique set and an inverse whose
canonical (sorted-rank) form equals the oracle's.  The plan's statistics,
written by the device at the end of each call, must report the batch size,
the keys that left stage 1 (per-tile distinct counts, computed here on the
host) and U; and its choice must follow them: batches whose tiles hold
almost no duplicates skip stage 1, duplicate-heavy ones keep it.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _check(orc, keys_np, uniq, inv, nu):
    U = int(nu.item())
    ref_u, ref_inv = orc.dedup(keys_np)
    u = to_np(uniq)[:U]
    assert U == ref_u.size and np.array_equal(np.sort(u), ref_u)
    if keys_np.size:
        i = to_np(inv)
        assert np.array_equal(u[i], keys_np)
        assert np.array_equal(np.searchsorted(ref_u, u[i]).astype(np.int32), ref_inv)


def _batches():
    rng = np.random.default_rng(42)
    yield "zipf", workloads.single_large_table(n=300_000).keys
    yield "distinct", rng.choice(1 << 50, 250_001, replace=False).astype(np.int64) - (1 << 49)
    yield "uniform", rng.integers(-5, 60_000, 200_003).astype(np.int64)
    yield "all_equal", np.full(70_000, -1, dtype=np.int64)
    yield "special", np.array([-1, -2, 0, np.iinfo(np.int64).max, np.iinfo(np.int64).min] * 999, dtype=np.int64)


@pytest.mark.parametrize("path", ["bins", "bins_only", "set"])
def test_each_stage2_form_matches_the_oracle(htl, orc, monkeypatch, path):
    monkeypatch.setenv("HTL_DEDUP_PATH", path)
    for name, keys_np in _batches():
        uniq, inv, nu = htl.dedup_unique_inverse(torch.from_numpy(keys_np).cuda())
        _check(orc, keys_np, uniq, inv, nu)


@pytest.mark.parametrize("n", [2049, 4096 + 17, (1 << 23)])
def test_bins_without_stage1_at_the_edges(htl, orc, monkeypatch, n):
    # a ragged last tile, and the largest batch the bins take
    monkeypatch.setenv("HTL_DEDUP_PATH", "bins_only")
    rng = np.random.default_rng(n)
    keys_np = rng.integers(0, max(n // 2, 1), n).astype(np.int64) * 1_000_003
    uniq, inv, nu = htl.dedup_unique_inverse(torch.from_numpy(keys_np).cuda())
    _check(orc, keys_np, uniq, inv, nu)


def _tile_survivors(keys_np, tile=2048):
    return sum(np.unique(keys_np[b:b + tile]).size for b in range(0, keys_np.size, tile))


def test_plan_statistics_and_choice(htl, orc):
    plan = htl.DedupPlan()
    assert plan.stats()["calls"] == 0
    assert plan.choose(1000) == htl.DEDUP_ONE_TILE
    assert plan.choose(1 << 20) == htl.DEDUP_TWO_STAGE_BINS     # nothing seen yet
    assert plan.choose((1 << 23) + 1) == htl.DEDUP_DEVICE_SET
    rng = np.random.default_rng(7)
    # 1) duplicate-heavy (Zipf): two stages, statistics as the host counts them
    z = workloads.single_large_table(n=1 << 20).keys
    uniq, inv, nu = plan.dedup(torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    _check(orc, z, uniq, inv, nu)
    st = plan.stats()
    assert st == {"calls": 1, "n": z.size, "survivors": _tile_survivors(z), "n_unique": np.unique(z).size,
                  "path": htl.DEDUP_TWO_STAGE_BINS}
    assert plan.choose(1 << 20) == htl.DEDUP_TWO_STAGE_BINS
    # 2) all distinct: still two stages (chosen from the Zipf batch), but its
    #    statistics (every key survives) send the next batch past stage 1
    d = rng.choice(1 << 60, 1 << 20, replace=False).astype(np.int64)
    uniq, inv, nu = plan.dedup(torch.from_numpy(d).cuda())
    torch.cuda.synchronize()
    _check(orc, d, uniq, inv, nu)
    st = plan.stats()
    assert st["calls"] == 2 and st["survivors"] == d.size and st["path"] == htl.DEDUP_TWO_STAGE_BINS
    assert plan.choose(1 << 20) == htl.DEDUP_BINS_ONLY
    d2 = rng.choice(1 << 60, 700_001, replace=False).astype(np.int64)
    uniq, inv, nu = plan.dedup(torch.from_numpy(d2).cuda())
    torch.cuda.synchronize()
    _check(orc, d2, uniq, inv, nu)
    st = plan.stats()
    assert st["calls"] == 3 and st["path"] == htl.DEDUP_BINS_ONLY
    assert st["survivors"] == d2.size and st["n_unique"] == d2.size
    # 3) duplicate-heavy again: calls 4..7 still skip stage 1 (the last
    #    measurement said the tiles hold no duplicates); call 8 runs both
    #    stages to measure again, and the plan goes back to two stages
    for call in range(4, 9):
        uniq, inv, nu = plan.dedup(torch.from_numpy(z).cuda())
        torch.cuda.synchronize()
        _check(orc, z, uniq, inv, nu)
        st = plan.stats()
        assert st["calls"] == call
        assert st["path"] == (htl.DEDUP_TWO_STAGE_BINS if call == 8 else htl.DEDUP_BINS_ONLY)
    assert st["survivors"] == _tile_survivors(z)
    assert plan.choose(1 << 20) == htl.DEDUP_TWO_STAGE_BINS
    # small and large batches report their own forms
    s = rng.integers(0, 300, 1500).astype(np.int64)
    uniq, inv, nu = plan.dedup(torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    _check(orc, s, uniq, inv, nu)
    assert plan.stats()["path"] == htl.DEDUP_ONE_TILE and plan.stats()["survivors"] == np.unique(s).size
    # an empty batch reports nothing
    e = np.zeros(0, dtype=np.int64)
    uniq, inv, nu = plan.dedup(torch.from_numpy(e).cuda())
    torch.cuda.synchronize()
    assert int(nu.item()) == 0 and plan.stats()["calls"] == 9
    plan.close()


def test_plan_on_a_large_batch_takes_the_device_set(htl, orc):
    plan = htl.DedupPlan()
    rng = np.random.default_rng(8)
    keys_np = rng.integers(0, 3_000_000, (1 << 23) + 5).astype(np.int64)
    uniq, inv, nu = plan.dedup(torch.from_numpy(keys_np).cuda())
    torch.cuda.synchronize()
    _check(orc, keys_np, uniq, inv, nu)
    st = plan.stats()
    assert st["path"] == htl.DEDUP_DEVICE_SET and st["n"] == keys_np.size
    assert st["survivors"] == _tile_survivors(keys_np)
    plan.close()


def test_plan_keeps_stage1_for_a_hot_key_among_distinct_ones(htl, orc):
    # 97% of the keys distinct, 3% one key spread over every tile: stage 1
    # keeps 97% of the keys, but without it that one key would put 3% of the
    # batch into a single bin -- the plan must keep both stages
    rng = np.random.default_rng(9)
    n = 1 << 20
    keys_np = rng.choice(1 << 60, n, replace=False).astype(np.int64)
    keys_np[rng.random(n) < 0.03] = 12345
    plan = htl.DedupPlan()
    for _ in range(3):
        uniq, inv, nu = plan.dedup(torch.from_numpy(keys_np).cuda())
        torch.cuda.synchronize()
        _check(orc, keys_np, uniq, inv, nu)
        assert plan.stats()["path"] == htl.DEDUP_TWO_STAGE_BINS
        assert plan.choose(n) == htl.DEDUP_TWO_STAGE_BINS
    assert plan.stats()["survivors"] == _tile_survivors(keys_np)
    plan.close()
