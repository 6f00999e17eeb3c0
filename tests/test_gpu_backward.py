"""GPU parity of the backward path: gradient segment-sum and row-wise Adam.

Segment sums are compared with the oracle's fp64 sums per element against
the recursive-summation error scale: |gpu - ref| <= 1e-5 * sum_i |g_i|
("1e-5 relative" read on the sum of magnitudes, since sums of N(0,1) values
cancel and the plain relative error of a near-zero sum is meaningless).  A
segment of one row must be copied exactly.

Adam is checked decoupled: the oracle's Adam is fed the GPU's own summed
gradient, and theta, m, v must agree within 1e-5 relative (plus a tiny
absolute floor for values near zero).
"""
import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _segsum_check(htl, orc, keys_np, grad_np):
    keys = torch.from_numpy(keys_np).cuda()
    grad = torch.from_numpy(grad_np).cuda()
    uniq, inv, nu = htl.dedup_unique_inverse(keys)
    U = int(nu.item())
    g = htl.segment_sum(grad, inv, nu, u_max=keys_np.size)
    got = to_np(g)[:U]
    inv_np = to_np(inv)
    ref, absum = orc.segment_sum(grad_np, inv_np, U)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * absum + 1e-30), float((err / np.maximum(absum, 1e-30)).max())
    counts = np.bincount(inv_np, minlength=U)
    single = counts == 1
    assert np.array_equal(got[single].astype(np.float64), ref[single])
    return uniq, inv, nu, g, U


@pytest.mark.parametrize("n,dim,spread", [(1, 4, 1), (5000, 16, 300), (70000, 128, 20000),
                                          (40000, 12, 50), (30000, 7, 3000), (9000, 256, 9000)])
def test_segment_sum_shapes(htl, orc, n, dim, spread):
    rng = np.random.default_rng(n + dim)
    keys = rng.integers(0, spread, n).astype(np.int64)
    grad = rng.standard_normal((n, dim)).astype(np.float32)
    _segsum_check(htl, orc, keys, grad)


def test_segment_sum_hot_segments(htl, orc):
    # one key holding 40% of the rows crosses the chunked long-segment path
    rng = np.random.default_rng(2)
    n, dim = 300_000, 32
    keys = np.where(rng.random(n) < 0.4, 7, rng.integers(0, 50_000, n)).astype(np.int64)
    keys[rng.random(n) < 0.1] = 11            # a second long segment
    grad = rng.standard_normal((n, dim)).astype(np.float32)
    _segsum_check(htl, orc, keys, grad)


def test_segment_sum_backward_workload_small(htl, orc):
    w = workloads.backward(n=1 << 17, dim=128)
    _segsum_check(htl, orc, w.keys, w.grad)


@pytest.mark.parametrize("dim,cap_log2", [(128, 18), (6, 16), (1028, 16)])
def test_adam_decoupled(htl, orc, dim, cap_log2):
    """Each step is checked from identical states: the oracle's array Adam gets
    the GPU table's theta, m, v before the step and the GPU's own summed
    gradient.  Tolerance: 1e-5 times the magnitudes of the terms each update
    adds (m and theta updates can cancel), so |err| <= 1e-5 * (|b1 m| + |(1-b1) g|)
    for m, likewise for v, and 1e-5 * (|theta| + |theta' - theta|) for theta."""
    w = workloads.backward(n=1 << 15, dim=dim, capacity_log2=cap_log2)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    table = htl.Table(w.capacity_log2, w.dim, "f32", adam=True)
    keys = torch.from_numpy(w.keys).cuda()
    grad = torch.from_numpy(w.grad).cuda()
    for step in (1, 2, 3):
        uniq, inv, nu = htl.dedup_unique_inverse(keys)
        U = int(nu.item())
        slots, status = table.find_or_insert(uniq, n_dev=nu, step=step)
        g = htl.segment_sum(grad, inv, nu, u_max=keys.numel())
        sl = to_np(slots)[:U]
        th0 = to_np(htl.table_tensor(table, "rows"))[sl]
        m0 = to_np(htl.table_tensor(table, "adam_m"))[sl]
        v0 = to_np(htl.table_tensor(table, "adam_v"))[sl]
        htl.rowwise_adam(table, slots[:U], g[:U], nu, lr, b1, b2, eps, step)
        th1 = to_np(htl.table_tensor(table, "rows"))[sl]
        m1 = to_np(htl.table_tensor(table, "adam_m"))[sl]
        v1 = to_np(htl.table_tensor(table, "adam_v"))[sl]
        gg = to_np(g)[:U]
        rth, rm, rv = orc.adam_arrays(th0, m0, v0, gg, lr, b1, b2, eps, step)
        d = np.float64
        tol_m = 1e-5 * (b1 * np.abs(m0.astype(d)) + (1 - b1) * np.abs(gg.astype(d))) + 1e-38
        tol_v = 1e-5 * (b2 * v0.astype(d) + (1 - b2) * gg.astype(d) ** 2) + 1e-38
        tol_t = 1e-5 * (np.abs(th0.astype(d)) + np.abs(rth.astype(d) - th0)) + 1e-38
        assert np.all(np.abs(m1.astype(d) - rm) <= tol_m)
        assert np.all(np.abs(v1.astype(d) - rv) <= tol_v)
        assert np.all(np.abs(th1.astype(d) - rth) <= tol_t)
        assert np.all(to_np(status)[:U] == (htl.INSERTED if step == 1 else htl.FOUND))


@pytest.mark.parametrize("dim", [128, 6])
def test_adam_bit_exact_against_fp32_oracle(htl, orc, dim):
    """The GPU's Adam (fp32, contraction off, correctly rounded division and
    square root) against the oracle's fp32 Adam in the same order, from
    identical states (the GPU table's theta, m, v and the GPU's summed
    gradient): theta, m and v bit for bit over three steps."""
    w = workloads.backward(n=1 << 14, dim=dim, capacity_log2=16)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    table = htl.Table(w.capacity_log2, w.dim, "f32", adam=True)
    keys = torch.from_numpy(w.keys).cuda()
    grad = torch.from_numpy(w.grad).cuda()
    for step in (1, 2, 3):
        uniq, inv, nu = htl.dedup_unique_inverse(keys)
        U = int(nu.item())
        slots, _ = table.find_or_insert(uniq, n_dev=nu, step=step)
        g = htl.segment_sum(grad, inv, nu, u_max=keys.numel())
        sl = to_np(slots)[:U]
        before = [to_np(htl.table_tensor(table, name))[sl] for name in ("rows", "adam_m", "adam_v")]
        htl.rowwise_adam(table, slots[:U], g[:U], nu, lr, b1, b2, eps, step)
        after = [to_np(htl.table_tensor(table, name))[sl] for name in ("rows", "adam_m", "adam_v")]
        want = orc.adam_arrays_f32(*before, to_np(g)[:U], lr, b1, b2, eps, step)
        for got, ref in zip(after, want):
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), step


def test_adam_closed_form_first_step(htl, orc):
    # from m = v = 0, step 1 moves theta by -lr * g / (|g| + eps)
    table = htl.Table(10, 8, "f32", adam=True)
    keys = torch.tensor([3, 9, 27], dtype=torch.int64, device="cuda")
    slots, _ = table.find_or_insert(keys)
    before = to_np(htl.gather(table, slots)).astype(np.float64)
    g = torch.tensor(np.random.default_rng(0).standard_normal((3, 8)), dtype=torch.float32, device="cuda")
    g[0, 0] = 0.0
    htl.rowwise_adam(table, slots, g, None, 1e-3, 0.9, 0.999, 1e-8, 1)
    after = to_np(htl.gather(table, slots)).astype(np.float64)
    gd = to_np(g).astype(np.float64)
    np.testing.assert_allclose(after, before - 1e-3 * gd / (np.abs(gd) + 1e-8), rtol=0, atol=3e-8)
    assert after[0, 0] == before[0, 0]


@pytest.mark.slow
def test_segment_sum_backward_full_size(htl, orc):
    """2^23 IDs, Zipf(1.2), dim 128: the full-size workload, every element checked."""
    w = workloads.backward()
    _segsum_check(htl, orc, w.keys, w.grad)


def _exact_grad(rng, n, dim):
    # multiples of 2^-6 in [-0.125, 0.125]: every fp32 sum of fewer than 2^17
    # of them is exact in any order, so the summed gradient does not depend
    # on the summation order and the fused and two-call paths see the same g
    return (rng.integers(-8, 9, (n, dim)) * 2.0 ** -6).astype(np.float32)


@pytest.mark.parametrize("dim,zipf", [(128, True), (16, True), (64, False), (6, True), (1028, False)])
def test_segment_sum_adam_fused_matches_two_calls(htl, orc, dim, zipf):
    """Fused segment-sum + Adam against segment_sum then rowwise_adam on a
    twin table: theta, m, v bit-equal over three steps (exact-sum gradients),
    and against the oracle's array Adam fed the oracle's segment sums."""
    rng = np.random.default_rng(dim)
    n = 1 << 15 if dim < 1024 else 1 << 12
    if zipf:
        keys_np = workloads.backward(n=n, dim=4, with_grad=False).keys
    else:
        keys_np = rng.integers(0, n // 3, n).astype(np.int64)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    fused = htl.Table(16, dim, "f32", adam=True)
    twin = htl.Table(16, dim, "f32", adam=True)
    keys = torch.from_numpy(keys_np).cuda()
    for step in (1, 2, 3):
        grad_np = _exact_grad(rng, n, dim)
        grad = torch.from_numpy(grad_np).cuda()
        uniq, inv, nu = htl.dedup_unique_inverse(keys)
        U = int(nu.item())
        slots, _ = fused.find_or_insert(uniq, n_dev=nu, step=step)
        slots2, _ = twin.find_or_insert(uniq, n_dev=nu, step=step)
        sl = to_np(slots)[:U]
        th0 = to_np(htl.table_tensor(fused, "rows"))[sl]
        m0 = to_np(htl.table_tensor(fused, "adam_m"))[sl]
        v0 = to_np(htl.table_tensor(fused, "adam_v"))[sl]
        htl.segment_sum_adam(fused, slots, grad, inv, nu, n, lr, b1, b2, eps, step)
        g = htl.segment_sum(grad, inv, nu, u_max=n)
        htl.rowwise_adam(twin, slots2[:U], g[:U], nu, lr, b1, b2, eps, step)
        sl2 = to_np(slots2)[:U]
        for name in ("rows", "adam_m", "adam_v"):
            a = to_np(htl.table_tensor(fused, name))[sl]
            b = to_np(htl.table_tensor(twin, name))[sl2]
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, step)
        # the oracle: exact segment sums, then its own Adam from the same state
        ref_g, _ = orc.segment_sum(grad_np, to_np(inv), U)
        rth, rm, rv = orc.adam_arrays(th0, m0, v0, ref_g.astype(np.float32), lr, b1, b2, eps, step)
        th1 = to_np(htl.table_tensor(fused, "rows"))[sl]
        d = np.float64
        assert np.array_equal(to_np(g)[:U].astype(d), ref_g)          # the sums are exact
        assert np.all(np.abs(to_np(htl.table_tensor(fused, "adam_m"))[sl].astype(d) - rm) <=
                      1e-5 * (b1 * np.abs(m0.astype(d)) + (1 - b1) * np.abs(ref_g)) + 1e-38)
        assert np.all(np.abs(th1.astype(d) - rth) <= 1e-5 * (np.abs(th0.astype(d)) + np.abs(rth - th0)) + 1e-38)
