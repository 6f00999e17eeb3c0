"""GPU tests at the largest sizes the C ABI accepts.

Slot numbers at the top of int32, row offsets past 2^32 bytes, a dedup batch
of 2^30 - 1 keys, a segment-sum of 2^31 - 1025 IDs and a pooled gather of
2^31 - 1 IDs: the oracle cannot run these, so each test checks what holds at
any size -- the closed-form initial rows of sampled keys (oracle), the unique
set against torch.unique, the identity unique[inverse[i]] == keys[i] for
every i, and segment and bag sums whose exact values follow from how the
inputs were built.  Tens of GB of device
memory each; the workspaces are released afterwards.
"""
import numpy as np
import pytest
import torch

from conftest import to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _release(htl):
    htl.release_workspaces()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_table_at_max_capacity(htl, orc):
    # 2^31 slots: slots reach the top of int32 and the rows span 32 GB
    table = htl.Table(31, 4, "f32")
    rng = np.random.default_rng(31)
    keys_np = np.unique(rng.integers(-(1 << 62), 1 << 62, 1 << 22)).astype(np.int64)
    keys = torch.from_numpy(keys_np).cuda()
    slots, st = table.find_or_insert(keys)
    assert (to_np(st) == htl.INSERTED).all()
    s = to_np(slots).astype(np.int64)
    assert s.min() >= 0 and s.max() < (1 << 31) and np.unique(s).size == s.size
    assert s.max() >= (1 << 30)                     # the upper half of the slots is in use
    slots2, st2 = table.find_or_insert(keys)
    assert (to_np(st2) == htl.FOUND).all() and np.array_equal(to_np(slots2), to_np(slots))
    rows = to_np(htl.gather(table, slots))          # one row per key
    pick = rng.choice(keys_np.size, 4096, replace=False)
    pick = np.concatenate([pick, np.argsort(s)[-64:]])   # and the highest slots
    assert np.array_equal(rows[pick], orc.init_rows(keys_np[pick], 4, orc.F32))
    assert (to_np(table.erase(keys[::2])) == htl.ERASED).all()
    _, st3 = table.find_or_insert(keys[1::2])
    assert (to_np(st3) == htl.FOUND).all()
    table.close()
    _release(htl)


def test_dedup_at_max_n(htl):
    n = (1 << 30) - 1                               # the largest batch dedup takes
    # keys drawn (by a multiplicative hash of the position) from 2^26 values
    i = torch.arange(n, dtype=torch.int64, device="cuda")
    x = i * 0x2545F4914F6CDD1D
    del i
    x = x ^ ((x >> 29) & ((1 << 35) - 1))
    x = x * 0x5851F42D4C957F2D
    keys = ((x >> 20) & ((1 << 26) - 1)) * 0x9E3779B97F4A7C1 - 12345
    del x
    uniq, inv, nu = htl.dedup_unique_inverse(keys)
    U = int(nu.item())
    want = torch.unique(keys)                       # sorted
    assert U == want.numel()
    assert torch.equal(torch.sort(uniq[:U])[0], want)
    del want
    assert int(inv.min().item()) >= 0 and int(inv.max().item()) < U
    assert torch.equal(uniq[inv.long()], keys)
    del uniq, inv, nu, keys
    _release(htl)


def test_segment_sum_at_max_n(htl):
    n = (1 << 31) - 1025                            # the largest n the segment-sum takes
    U, dim = 1 << 20, 4
    grad = torch.empty((n, dim), dtype=torch.float32, device="cuda")
    inv = torch.empty(n, dtype=torch.int32, device="cuda")
    step = 1 << 28
    for b in range(0, n, step):                     # id i: segment i mod U, row (i mod 7) + j
        e = min(n, b + step)
        i = torch.arange(b, e, dtype=torch.int64, device="cuda")
        inv[b:e] = (i % U).to(torch.int32)
        grad[b:e] = (i % 7).to(torch.float32)[:, None] + torch.arange(dim, dtype=torch.float32, device="cuda")
        del i
    nu = torch.tensor([U], dtype=torch.int64, device="cuda")
    g = to_np(htl.segment_sum(grad, inv, nu, u_max=U))
    del grad, inv
    # segment u holds i = u + kU for k < K_u; U = 4 (mod 7), so (u + kU) mod 7
    # runs through all seven residues every seven k: the sums are exact
    u = np.arange(U, dtype=np.int64)
    K = (n - 1 - u) // U + 1
    S = 21 * (K // 7)
    for r in range(6):
        S += np.where(K % 7 > r, (u + r * U) % 7, 0)
    want = S[:, None].astype(np.float64) + np.arange(dim)[None, :] * K[:, None]
    assert np.array_equal(g.astype(np.float64), want)
    _release(htl)


def test_pooling_at_max_n(htl, orc):
    # 2^31 - 1 IDs in 2^16 bags, the last ending at the top of int32: each
    # ID i reads the row of key i mod 64 of a bf16 table, so a bag's sum is
    # a count-weighted sum of 64 rows, exact in fp32 (bag lengths <= 2^16)
    n, nbags, U, dim = (1 << 31) - 1, 1 << 16, 64, 8
    table = htl.Table(10, dim, "bf16")
    keys_np = np.arange(U, dtype=np.int64) * 7919 + 3
    slots, st = table.find_or_insert(torch.from_numpy(keys_np).cuda())
    assert (to_np(st) == htl.INSERTED).all()
    inv = torch.empty(n, dtype=torch.int32, device="cuda")
    step = 1 << 28
    for b in range(0, n, step):
        e = min(n, b + step)
        inv[b:e] = (torch.arange(b, e, dtype=torch.int64, device="cuda") % U).to(torch.int32)
    rng = np.random.default_rng(7)
    offsets_np = np.linspace(0, n, nbags + 1).round().astype(np.int64)   # bags of ~32768 IDs
    offsets_np[1:-1] += rng.integers(-2000, 2001, nbags - 1)
    assert offsets_np[-1] == n and np.diff(offsets_np).min() > 0 and np.diff(offsets_np).max() <= 1 << 16
    offsets = torch.from_numpy(offsets_np.astype(np.int32)).cuda()
    out = to_np(htl.gather_pool(table, slots, inv, offsets, out_dtype="f32"))
    del inv
    # count of i in [a, e) with i mod U == r, for every bag and r
    r = np.arange(U, dtype=np.int64)[None, :]
    a, e = offsets_np[:-1, None], offsets_np[1:, None]
    cnt = (e - 1 - r) // U - (a - 1 - r) // U
    rows = orc.bf16_bits_to_f32(orc.init_rows(keys_np, dim, orc.BF16)).astype(np.float64)
    want = cnt.astype(np.float64) @ rows
    assert np.array_equal(out.astype(np.float64), want)
    table.close()
    _release(htl)
