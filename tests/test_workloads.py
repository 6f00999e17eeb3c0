"""Checks of the seeded input generators (shapes, distributions, encodings).

The generators stand in for Meituan's proprietary logs (MTGR, arXiv
2505.18654, section 6.1).  Pins: scramble is a bijection (exhaustive at small
k); Zipf frequencies of the head ranks match r^-a / H; the number of unique
keys and the pre-fill hit rate match their expectations
E[U] = sum_r 1 - (1 - p_r)^N and sum_{r <= P} p_r, computed here from the
Zipf law itself (an integral for the far tail); merged keys decode to
(table, id) with id below the table's vocabulary.
"""
import math

import numpy as np
import pytest
from scipy import integrate

import workloads


def test_scramble_is_a_bijection():
    for k in (1, 2, 5, 8, 13, 16):
        x = np.arange(1 << k, dtype=np.uint64)
        y = workloads.scramble(x, k)
        assert np.all(y < (1 << k))
        assert np.unique(y).size == 1 << k
    big = workloads.scramble(np.arange(1 << 16, dtype=np.uint64), 40)
    assert np.unique(big).size == 1 << 16 and np.all(big < (1 << 40))


def _zipf_pmf_head(a, K, R):
    r = np.arange(1, R + 1, dtype=np.float64)
    head = r ** -a
    tail = 0.0
    if K > R:   # midpoint rule tail: integral of x^-a from R + 0.5 to K + 0.5
        tail = ((R + 0.5) ** (1 - a) - (K + 0.5) ** (1 - a)) / (a - 1)
    return head, head.sum() + tail


def _expected_unique(a, K, N, R=1 << 21):
    head, H = _zipf_pmf_head(a, K, min(K, R))
    p = head / H
    e = float(np.sum(-np.expm1(N * np.log1p(-p))))
    if K > R:
        c = N / H
        f = lambda y: -math.expm1(-c * math.exp(-a * y)) * math.exp(y)
        tail, _ = integrate.quad(f, math.log(R + 0.5), math.log(K + 0.5), limit=400)
        e += tail
    return e


def test_zipf_head_frequencies():
    rng = np.random.Generator(np.random.PCG64(11))
    a, K, n = 1.1, 1 << 20, 400_000
    r = workloads.zipf_ranks(rng, a, K, n)
    assert r.min() >= 1 and r.max() <= K
    head, H = _zipf_pmf_head(a, K, K)
    counts = np.bincount(r, minlength=11)[1:11]
    exp = n * head[:10] / H
    assert np.all(np.abs(counts - exp) < 5 * np.sqrt(exp))


def test_tiny_unique_count_matches_expectation():
    w = workloads.tiny()
    assert w.keys.dtype == np.int64 and w.keys.size == 65536
    assert w.keys.min() >= 0 and w.keys.max() < (1 << 20)
    U = np.unique(w.keys).size
    E = _expected_unique(1.1, 1 << 20, 65536)
    assert abs(E - 17311) < 20                 # the expectation itself
    assert abs(U - E) < 5 * math.sqrt(E)


@pytest.mark.slow
def test_single_large_table_hit_rate_and_unique_count():
    w = workloads.single_large_table()
    N, P = w.keys.size, w.prefill.size
    assert N == 1 << 22 and P == 1 << 23 and w.capacity_log2 == 24 and w.dim == 64
    assert np.unique(w.prefill).size == P
    hit = np.isin(w.keys, w.prefill)
    head, H = _zipf_pmf_head(1.05, 1 << 40, P)
    p_hit = head.sum() / H
    assert abs(p_hit - 0.7425) < 0.002
    assert abs(hit.mean() - p_hit) < 5 * math.sqrt(p_hit * (1 - p_hit) / N) + 0.002
    U = np.unique(w.keys).size
    E = _expected_unique(1.05, 1 << 40, N)
    assert abs(U - E) < 5 * math.sqrt(E) + 0.002 * E


def test_merged_tables_layout():
    w = workloads.merged_tables(batch=600)
    nt = 26
    vocab = workloads.merged_vocab_sizes()
    assert vocab[0] == 1000 and vocab[-1] == 10**8 and vocab.size == nt
    assert w.nbags == 600 * nt and w.offsets.size == w.nbags + 1
    assert w.offsets[0] == 0 and w.offsets[-1] == w.keys.size
    lens = np.diff(w.offsets)
    assert abs(lens.mean() - 20) < 0.5
    table = (w.keys >> 48).astype(np.int64)
    ids = w.keys & ((1 << 48) - 1)
    bag_table = np.repeat(np.tile(np.arange(nt), 600), lens)
    assert np.array_equal(table, bag_table)
    assert np.all(ids < vocab[table])


def test_backward_shapes():
    w = workloads.backward(n=4096, dim=32)
    assert w.grad.shape == (4096, 32) and w.grad.dtype == np.float32
    assert abs(w.grad.mean()) < 0.02 and abs(w.grad.std() - 1) < 0.02
    again = workloads.backward(n=4096, dim=32)
    assert np.array_equal(again.keys, w.keys) and np.array_equal(again.grad, w.grad)


def test_dynamic_online_window_drifts():
    spec = workloads.DynamicOnlineSpec(window=1 << 12, n=1 << 12, steps=5)
    inv_keys = {}
    for s in range(3):
        keys = workloads.dynamic_online_step(spec, s)
        assert keys.size == spec.n
        lo = s * spec.delta
        allowed = workloads.scramble(np.arange(lo, lo + spec.window, dtype=np.uint64), 40)
        assert np.all(np.isin(keys, allowed.astype(np.int64)))
        inv_keys[s] = set(allowed.tolist())
    assert len(inv_keys[1] - inv_keys[0]) == spec.delta


def test_dynamic_online_stream_matches_per_step_definition():
    spec = workloads.DynamicOnlineSpec(window=1 << 12, n=1 << 10, steps=6)
    stream = workloads.DynamicOnlineStream(spec, 6)
    for s in (0, 1, 5):
        assert np.array_equal(stream.keys(s), workloads.dynamic_online_step(spec, s))
