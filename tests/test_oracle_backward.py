"""Pins for the oracle's backward path: gradient segment-sum and row-wise Adam.

Segment sum (backward gradient dedup): g_u = sum of grad[i] over the IDs i
whose key is unique key u, accumulated in fp64.  Pins: numpy.add.at in fp64
(an independent library routine, same order, so equal bits); the
permutation case U = N (every segment one row: the sum is the row itself);
math.fsum on a single long segment within fp64's rounding bound.

Adam (Kingma & Ba, Algorithm 1; the TensorFlow page, section 3.2, keeps
Adam's beta terms on every parameter server): pins are closed forms of the
bias-corrected update.  From m = v = 0 with a constant gradient g, m_t/(1-b1^t)
= g and v_t/(1-b2^t) = g^2 at every step, so each step moves theta by
-lr * g / (|g| + eps) exactly; a dropped or wrong bias correction breaks this.
Rows that are not in the batch do not change; a zero gradient at t = 1 leaves
theta unchanged.
"""
import math

import numpy as np


def test_segment_sum_matches_numpy_add_at(orc):
    rng = np.random.default_rng(0)
    n, d, U = 5000, 16, 300
    inv = rng.integers(0, U, n).astype(np.int32)
    g = rng.standard_normal((n, d)).astype(np.float32)
    s, a = orc.segment_sum(g, inv, U)
    ref = np.zeros((U, d))
    np.add.at(ref, inv, g.astype(np.float64))
    aref = np.zeros((U, d))
    np.add.at(aref, inv, np.abs(g.astype(np.float64)))
    assert np.array_equal(s, ref)
    assert np.array_equal(a, aref)


def test_segment_sum_permutation_and_single_segment(orc):
    rng = np.random.default_rng(1)
    n, d = 777, 8
    g = rng.standard_normal((n, d)).astype(np.float32)
    perm = rng.permutation(n).astype(np.int32)
    s, _ = orc.segment_sum(g, perm, n)
    assert np.array_equal(s[perm], g.astype(np.float64))
    s1, a1 = orc.segment_sum(g, np.zeros(n, np.int32), 1)
    for j in range(d):
        exact = math.fsum(g[:, j].astype(np.float64))
        assert abs(s1[0, j] - exact) <= n * 2.0**-53 * a1[0, j]


def test_adam_constant_gradient_closed_form(orc):
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    t = orc.Table(64, 6, orc.F32, adam=True)
    keys = np.array([10, 20], np.int64)
    t.find_or_insert(keys)
    theta0 = {int(k): t.lookup(k)[0].astype(np.float64) for k in keys}
    g = np.array([[0.5, -2.0, 1e-3, -1e-6, 3.0, 0.0]] * 2, np.float32)
    steps = 5
    for s in range(1, steps + 1):
        t.adam(keys, g, lr, b1, b2, eps, step=s)
    gd = g[0].astype(np.float64)
    move = lr * gd / (np.abs(gd) + eps)
    for k in keys:
        row, _, m, v = t.lookup(k)
        want = theta0[int(k)] - steps * move
        assert np.allclose(row, want, rtol=0, atol=4e-8), (row, want)
        # first and second moments after `steps` constant-gradient updates
        bf1, bf2 = np.float64(np.float32(b1)), np.float64(np.float32(b2))
        assert np.allclose(m, (1 - bf1**steps) * gd, rtol=1e-6, atol=1e-12)
        assert np.allclose(v, (1 - bf2**steps) * gd * gd, rtol=1e-6, atol=1e-18)


def test_adam_touches_only_batch_rows_and_zero_grad_is_noop(orc):
    t = orc.Table(64, 4, orc.F32, adam=True)
    t.find_or_insert([1, 2, 3])
    before = {k: t.lookup(k)[0].copy() for k in (1, 2, 3)}
    g = np.zeros((1, 4), np.float32)
    g[0, 1] = 1.0
    t.adam(np.array([2], np.int64), g, step=1)
    assert np.array_equal(t.lookup(1)[0], before[1])
    assert np.array_equal(t.lookup(3)[0], before[3])
    r2 = t.lookup(2)[0]
    assert r2[0] == before[2][0] and r2[2] == before[2][2]
    assert r2[1] != before[2][1]
    t.adam(np.array([999], np.int64), g, step=1)     # not live: ignored
    assert len(t) == 3


def test_adam_array_form_matches_table_form(orc):
    rng = np.random.default_rng(8)
    t = orc.Table(64, 8, orc.F32, adam=True)
    keys = np.array([4, 5, 6], np.int64)
    t.find_or_insert(keys)
    th = np.stack([t.lookup(k)[0] for k in keys])
    m = np.zeros_like(th)
    v = np.zeros_like(th)
    for step in (1, 2, 3, 4):
        g = rng.standard_normal(th.shape).astype(np.float32)
        t.adam(keys, g, step=step)
        th, m, v = orc.adam_arrays(th, m, v, g, step=step)
        for i, k in enumerate(keys):
            row, _, mk, vk = t.lookup(k)
            assert np.array_equal(row, th[i]) and np.array_equal(mk, m[i]) and np.array_equal(vk, v[i])


def test_adam_f32_within_fp32_rounding_of_the_fp64_adam(orc):
    # the fp32 evaluation and the fp64 one agree to within the rounding of
    # the few fp32 operations each value goes through (2^-24 each, relative to
    # the terms that make it up), over three steps from random states
    rng = np.random.default_rng(11)
    n = 50_000
    th = rng.normal(0, 0.1, n).astype(np.float32)
    m = rng.normal(0, 0.01, n).astype(np.float32)
    v = np.abs(rng.normal(0, 1e-4, n)).astype(np.float32)
    u = 2.0 ** -24
    for step in (1, 2, 7):
        g = rng.normal(0, 1, n).astype(np.float32)
        t32, m32, v32 = orc.adam_arrays_f32(th, m, v, g, step=step)
        t64, m64, v64 = orc.adam_arrays(th, m, v, g, step=step)
        d = np.float64
        assert np.all(np.abs(m32.astype(d) - m64) <= 4 * u * (0.9 * np.abs(m.astype(d)) + 0.1 * np.abs(g.astype(d))))
        assert np.all(np.abs(v32.astype(d) - v64) <= 4 * u * (0.999 * v.astype(d) + 0.001 * g.astype(d) ** 2))
        assert np.all(np.abs(t32.astype(d) - t64) <= 16 * u * (np.abs(th.astype(d)) + np.abs(t64.astype(d) - th)))
        # and they do differ somewhere: the evaluation really is fp32
        assert not np.array_equal(t32, t64)
        th, m, v = t32, m32, v32


def test_adam_f32_first_step_closed_form(orc):
    # from m = v = 0 at t = 1: m/c1 = g and v/c2 = g^2 up to rounding, so
    # theta moves by lr * g / (|g| + eps); a zero gradient moves nothing
    rng = np.random.default_rng(12)
    g = rng.normal(0, 1, 20_000).astype(np.float32)
    g[:5] = 0.0
    th = rng.normal(0, 0.1, g.size).astype(np.float32)
    z = np.zeros_like(g)
    t1, m1, v1 = orc.adam_arrays_f32(th, z, z, g, lr=1e-3, step=1)
    want = th.astype(np.float64) - 1e-3 * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + 1e-8)
    np.testing.assert_allclose(t1, want, rtol=0, atol=3e-8)
    assert np.array_equal(t1[:5], th[:5]) and not m1[:5].any() and not v1[:5].any()
