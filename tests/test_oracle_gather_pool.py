"""Pins for the oracle's row gather and bag sum-pooling.

Row gather is the lookup itself (MTGenRec TL;DR, "faster embedding
lookups"): out[i] is a copy of the row of keys[i].  Sum pooling over
multi-hot bags is this build's reading for bag-shaped inputs (the pages do not
describe pooling): fp64 sum over the bag, rounded to fp32 and, for bf16
output, from there to bf16 (nearest even); empty bags give zeros.

Pins: gathered rows equal the closed-form rows; pooled sums equal an
independent numpy fp64 recomputation from the gathered rows; for bf16 rows
the fp32 partial sums of any order are exact (every bf16 row value is a
multiple of 2^-10 with |value| <= 1/8, so sums of up to 2^16 of them need at
most 24 significant bits), which the test checks against a random order; the
bf16 output equals torch's round-to-nearest-even of the fp32 sum.
"""
import numpy as np
import torch


def _table_with(orc, keys, dim, dtype):
    t = orc.Table(1 << 16, dim, dtype=dtype)
    t.find_or_insert(np.unique(keys))
    return t


def test_gather_copies_closed_form_rows(orc):
    import workloads
    keys = workloads.tiny(n=3000).keys
    for dtype in (orc.F32, orc.BF16):
        t = _table_with(orc, keys, 16, dtype)
        out = t.gather(keys)
        assert np.array_equal(out, orc.init_rows(keys, 16, dtype))
        missing = t.gather(np.array([123456789012], dtype=np.int64))
        assert not missing.any()


def test_pool_matches_numpy_and_is_order_free(orc):
    rng = np.random.default_rng(4)
    nb = 400
    lens = rng.poisson(20, nb)
    lens[:5] = 0                                          # empty bags
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    keys = rng.integers(0, 3000, offsets[-1]).astype(np.int64) | (np.int64(3) << 48)
    t = _table_with(orc, keys, 24, orc.BF16)
    rows = orc.bf16_bits_to_f32(t.gather(keys)).astype(np.float64)
    ref = np.zeros((nb, 24))
    for b in range(nb):
        ref[b] = rows[offsets[b]:offsets[b + 1]].sum(axis=0)
    p32 = t.gather_pool(keys, offsets, orc.F32)
    assert np.array_equal(p32.astype(np.float64), ref)     # exact: no rounding happened
    assert not p32[:5].any()
    # any fp32 summation order gives the same bits
    for b in rng.integers(0, nb, 20):
        seg = rows[offsets[b]:offsets[b + 1]].astype(np.float32)
        acc = np.zeros(24, np.float32)
        for r in seg[rng.permutation(seg.shape[0])]:
            acc = acc + r
        assert np.array_equal(acc, p32[b])
    pbf = t.gather_pool(keys, offsets, orc.BF16)
    want = torch.from_numpy(p32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pbf, want)


def test_pool_fp32_rows_within_rounding(orc):
    rng = np.random.default_rng(5)
    offsets = np.arange(0, 41 * 50, 41, dtype=np.int32)
    keys = rng.integers(0, 500, offsets[-1]).astype(np.int64)
    t = _table_with(orc, keys, 8, orc.F32)
    rows = t.gather(keys).astype(np.float64)
    ref = np.add.reduceat(rows, offsets[:-1], axis=0)
    got = t.gather_pool(keys, offsets, orc.F32).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0**-24 * np.abs(ref) + 1e-45)


def test_pool_skips_keys_that_are_not_live(orc):
    t = orc.Table(64, 4)
    t.find_or_insert([1, 2])
    out = t.gather_pool(np.array([1, 999, 2], np.int64), np.array([0, 3], np.int32))
    assert np.array_equal(out[0], (orc.init_row(1, 4).astype(np.float64)
                                   + orc.init_row(2, 4)).astype(np.float32))
