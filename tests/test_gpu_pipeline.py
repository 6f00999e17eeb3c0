"""The copy / lookup / compute pipeline (LookupPipeline) on the GPU: every
batch that leaves it matches the oracle table stepped batch by batch --
statuses, gathered rows, pooled bags -- while the next batches are copied
and looked up on their own streams, and a caller that holds each batch's
outputs on a busy stream never sees them overwritten."""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _stream_batches(sizes, seed=0):
    rng = np.random.default_rng(seed)
    for n in sizes:
        r = workloads.zipf_ranks(rng, 1.1, 1 << 18, n) if n else np.zeros(0, dtype=np.int64)
        yield workloads.scramble(r - 1, 18).astype(np.int64) if n else r


@pytest.mark.parametrize("depth", [2, 3])
def test_pipeline_batches_match_the_oracle(htl, orc, depth):
    sizes = [5000, 70_000, 0, 1, 2048, 2049, 123_457, 70_000, 9, 100_000]
    batches = list(_stream_batches(sizes))
    table = htl.Table(17, 16, "f32", last_seen=True)
    otab = orc.Table(1 << 17, 16, orc.F32)
    pipe = htl.LookupPipeline(table, n_max=max(sizes), depth=depth)
    seen = 0
    for b in pipe.run(batches, step0=3, steps_per_batch=2):
        keys_np = batches[b.index]
        U = int(b.n_unique.item())
        u = to_np(b.unique)[:U]
        assert np.array_equal(np.sort(u), np.unique(keys_np))
        if keys_np.size:
            assert np.array_equal(u[to_np(b.inverse)[:keys_np.size]], keys_np)
        assert np.array_equal(to_np(b.status)[:U], otab.find_or_insert(u, step=3 + 2 * b.index))
        assert np.array_equal(to_np(b.out), otab.gather(keys_np))
        seen += 1
    assert seen == len(sizes)
    # last_seen follows the steps the pipeline stamped
    k, ls, _, n = table.scan()
    L = int(n.item())
    ok, ols = otab.live()
    order = np.argsort(to_np(k)[:L])
    assert np.array_equal(to_np(k)[:L][order], ok)
    assert np.array_equal(to_np(ls)[:L][order].astype(np.uint32), ols)


def test_pipeline_with_a_slow_consumer(htl, orc):
    # the caller keeps each batch busy on its own stream before reading it:
    # the lookup two batches later must wait for it, not overwrite the rows
    sizes = [40_000] * 8
    batches = list(_stream_batches(sizes, seed=5))
    table = htl.Table(17, 32, "bf16")
    otab = orc.Table(1 << 17, 32, orc.BF16)
    pipe = htl.LookupPipeline(table, n_max=max(sizes))
    copies = []
    for b in pipe.run(batches):
        torch.cuda._sleep(2_000_000)            # the caller's stream is busy first
        copies.append((b.index, b.out.clone()))
    torch.cuda.synchronize()
    for i, out in copies:
        keys_np = batches[i]
        otab.find_or_insert(np.unique(keys_np))
        assert np.array_equal(to_np(out), otab.gather(keys_np)), i


def test_pipeline_pooled_bags(htl, orc):
    m = [workloads.merged_tables(seed=s, batch=512, capacity_log2=20) for s in range(4)]
    table = htl.Table(20, m[0].dim, "bf16")           # room for every key of the four batches
    otab = orc.Table(1 << 20, m[0].dim, orc.BF16)
    pipe = htl.LookupPipeline(table, n_max=max(w.keys.size for w in m), nbags_max=max(w.nbags for w in m))
    items = [(w.keys, torch.from_numpy(w.offsets).cuda()) for w in m]
    for b in pipe.run(items):
        w = m[b.index]
        U = int(b.n_unique.item())
        assert np.array_equal(to_np(b.status)[:U], otab.find_or_insert(to_np(b.unique)[:U], step=b.index))
        assert np.array_equal(to_np(b.out), otab.gather_pool(w.keys, w.offsets, orc.BF16))
