"""Pins for the oracle's closed-form row initialisation and bf16 rounding.

The pages give no initialiser; the reading is "row values initialised by a
seeded hash of (table id, key)", where the table id travels inside the merged
64-bit key (MTGenRec, "automatic table merging").  The oracle builds a row
from a SplitMix64 stream (Steele, Lea & Flood 2014) seeded with
mix64(key ^ mix64(seed)).

Pins: the SplitMix64 known-answer vector of the reference implementation
(tests/golden/splitmix64_seed1234567.txt); the value lattice and range that
make fp32 and bf16 rows exact; the relation between the bf16 and fp32 rows of
one key (both come from the same 32-bit words); uniformity of the codes; and
torch's float->bfloat16 conversion (round to nearest even) for the rounding.
"""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed1234567.txt")


def _golden():
    with open(GOLDEN) as f:
        return [int(line) for line in f if line.strip() and not line.startswith("#")]


def test_splitmix64_known_answer(orc):
    assert orc.splitmix64(1234567, 5).tolist() == _golden()


def test_mix64_fixed_point_and_spread(orc):
    assert orc.mix64(0) == 0            # every step of the finaliser maps 0 to 0
    vals = {orc.mix64(i) for i in range(1, 4097)}
    assert len(vals) == 4096            # a bijection never collides


def test_row_words_come_from_the_splitmix_stream(orc):
    for key in (0, 1, -5, 123456789, (7 << 48) | 99):
        for seed in (0, 3):
            base = orc.mix64((key & 0xFFFFFFFFFFFFFFFF) ^ orc.mix64(seed))
            words = orc.splitmix64(base, 4)
            row = orc.init_row(key, 8, orc.F32, seed)
            codes = np.rint(row.astype(np.float64) * 2.0**26).astype(np.int64) + (1 << 23)
            hi = (words >> np.uint64(32)).astype(np.int64)
            lo = (words & np.uint64(0xFFFFFFFF)).astype(np.int64)
            expect = np.stack([hi, lo], axis=1).reshape(-1) >> 8
            assert np.array_equal(codes, expect)


def test_lattice_range_and_exactness(orc):
    keys = np.random.default_rng(0).integers(-(2**62), 2**62, 3000)
    f = orc.init_rows(keys, 16, orc.F32)
    b = orc.bf16_bits_to_f32(orc.init_rows(keys, 16, orc.BF16))
    for arr, step in ((f, 2.0**-26), (b, 2.0**-10)):
        a = arr.astype(np.float64)
        assert a.min() >= -0.125 and a.max() < 0.125
        q = a / step
        assert np.array_equal(q, np.rint(q))
    # the bf16 value keeps the top 8 of the fp32 value's 24 code bits
    assert np.array_equal(b.astype(np.float64), np.floor(f.astype(np.float64) * 1024.0) / 1024.0)


def test_codes_look_uniform(orc):
    keys = np.arange(4000, dtype=np.int64)
    f = orc.init_rows(keys, 32, orc.F32).astype(np.float64).reshape(-1)
    n = f.size
    assert abs(f.mean()) < 5 * (0.25 / np.sqrt(12)) / np.sqrt(n)
    assert abs(f.var() - 0.25**2 / 12) < 0.02 * 0.25**2 / 12
    top = np.floor((f + 0.125) * 64).astype(np.int64)          # 16 equal bins
    counts = np.bincount(top, minlength=16)
    chi2 = ((counts - n / 16) ** 2 / (n / 16)).sum()
    assert chi2 < 60                                          # 15 dof, p ~ 1e-7


def test_keys_and_seeds_give_distinct_rows(orc):
    r = {orc.init_row(k, 8).tobytes() for k in range(2000)}
    assert len(r) == 2000
    assert not np.array_equal(orc.init_row(5, 8, seed=0), orc.init_row(5, 8, seed=1))
    assert np.array_equal(orc.init_row(5, 8, seed=9), orc.init_row(5, 8, seed=9))
    # a longer row extends a shorter one
    assert np.array_equal(orc.init_row(77, 64)[:16], orc.init_row(77, 16))


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 100,
        # exact ties between two bf16 values, both parities of the kept bit
        (np.arange(1, 500, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, np.inf, -np.inf], dtype=np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16_bits(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
