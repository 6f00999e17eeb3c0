"""Pins for the oracle's probe-coverage functions (MTGenRec, Theorem 1).

Theorem 1 of MTGenRec (arXiv 2505.12663): in a table of M = 2^n slots, the
probe sequence h_t = (h0 + t*S) mod M, t = 0..M-1, visits all M slots exactly
when the step S is odd.  The page's statement is garbled (it calls S odd in
the premise as well); the reading used here is "S arbitrary, full coverage
iff S odd".  The truncated "Formally:" part and the unprinted Lemma 1 are read
as the elementary fact behind it: t*S = t'*S (mod M) iff t = t'
(mod M / gcd(S, M)), so the walk visits exactly M / gcd(S mod M, M) slots,
with gcd(0, M) = M.

The oracle counts visited slots by brute force; these tests hold it to that
closed form for every step S in [0, 2M) at M = 2^1 .. 2^12, from several
starting slots, and to the bucketed form the GPU table uses (the same walk
over M/W buckets of W consecutive slots).
"""
import math

import numpy as np
import pytest


def _starts(M, rng):
    return sorted({0, 1 % M, M - 1, *[int(x) for x in rng.integers(0, M, 3)]})


def test_closed_form_every_step_every_size(orc):
    rng = np.random.default_rng(12345)
    for n in range(1, 13):
        M = 1 << n
        for h0 in _starts(M, rng):
            for S in range(0, 2 * M):
                got = orc.probe_coverage(M, h0, S)
                g = math.gcd(S % M, M)        # gcd(0, M) = M
                assert got == M // g, (M, h0, S, got)
                assert (got == M) == (S % 2 == 1), (M, h0, S)


def test_even_steps_cover_a_strict_subset(orc):
    # S = 2^j * odd covers M / 2^j slots, i.e. a strict subset for j >= 1.
    M = 1 << 10
    for j in range(1, 11):
        for odd in (1, 3, 5, 7, 1023):
            S = ((1 << j) * odd) % (2 * M)
            expect = M // math.gcd(S % M, M)
            assert orc.probe_coverage(M, 17, S) == expect
            assert expect < M


@pytest.mark.parametrize("W", [1, 2, 4, 8, 16])
def test_bucketed_walk_covers_all_slots_iff_odd_bucket_step(orc, W):
    rng = np.random.default_rng(7)
    for n in range(0, 11):
        M = W << n           # n buckets-log2, so M/W = 2^n buckets
        nb = M // W
        for b0 in _starts(nb, rng):
            for S in range(0, 2 * nb):
                got = orc.bucket_probe_coverage(M, W, b0, S)
                expect = W * (nb // math.gcd(S % nb, nb))
                assert got == expect, (M, W, b0, S, got)
                if nb >= 2:
                    assert (got == M) == (S % 2 == 1)
                else:
                    assert got == M
