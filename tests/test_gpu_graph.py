"""The forward lookup captured in a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls) and replayed: every replay, with eager work and synchronisations
between replays, must give what the eager calls give.

A fixed table's dedup, find-or-insert and gather only launch kernels on the
caller's stream (no allocation, no memset, no synchronisation once the dedup
workspace exists), so the whole step can be captured.  The table's key array
is restored between replays, as the benchmark does, so every replay starts
from the same table.
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # workspaces exist before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = step()
    return g, res


def _by_key(u, vals):
    return dict(zip(u.tolist(), vals.tolist()))


@pytest.mark.parametrize("pooled", [False, True])
def test_lookup_graph_replays_match_eager(htl, orc, pooled):
    if pooled:
        w = workloads.merged_tables(batch=2048, capacity_log2=20)   # 303,759 keys
        offsets = torch.from_numpy(w.offsets).cuda()
    else:
        w = workloads.tiny(n=100_000)
        offsets = None
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    keys = torch.from_numpy(w.keys).cuda()
    saved = htl.table_keys(table).clone()
    view = table.view()

    def restore():
        htl._binding.copy_to_device_ptr(view.keys, saved)

    def step():
        return htl.lookup(table, keys, offsets=offsets, out_dtype="bf16" if pooled else None)

    out_e, uniq_e, inv_e, nu_e, slots_e, st_e = step()
    U = int(nu_e.item())
    ref_out = to_np(out_e).copy()
    ref_u = to_np(uniq_e)[:U].copy()
    ref_st = _by_key(ref_u, to_np(st_e)[:U])
    restore()
    g, (out, uniq, inv, nu, slots, status) = _capture(step)

    other = htl.Table(12, 8, "f32")
    rng = np.random.default_rng(0)
    for rep in range(5):
        restore()
        # eager work between replays, on the same stream, then a synchronisation
        htl.lookup(other, torch.from_numpy(rng.integers(0, 1 << 20, 5000).astype(np.int64)).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Ur = int(nu.item())
        u = to_np(uniq)[:Ur]
        assert Ur == U and np.array_equal(np.sort(u), np.sort(ref_u)), rep
        assert np.array_equal(u[to_np(inv)], w.keys), rep
        assert _by_key(u, to_np(status)[:Ur]) == ref_st, rep
        assert np.array_equal(to_np(out), ref_out), rep
    # and the replayed rows are the oracle's
    otab = orc.Table(1 << w.capacity_log2, w.dim, orc.F32 if w.dtype == "f32" else orc.BF16)
    otab.find_or_insert(ref_u)
    if pooled:
        assert np.array_equal(to_np(out), otab.gather_pool(w.keys, w.offsets, orc.BF16))
    else:
        assert np.array_equal(to_np(out), otab.gather(w.keys))
