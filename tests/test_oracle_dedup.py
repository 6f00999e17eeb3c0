"""Pins for the oracle's feature-ID dedup (unique + inverse).

MTGenRec (arXiv 2505.12663), TL;DR: two-stage ID deduplication speeds up
embedding lookups; MTGR (arXiv 2505.18654) section 5, "Embedding Lookup": IDs
stay unique before and after the all-to-all.  Whatever the stages, the result
is the plain unique-with-inverse of the batch.  The oracle's sorted form is
held to numpy.unique (an independent library routine), to the defining
invariants, and to the special cases N = 0, all-equal and all-distinct.
"""
import numpy as np
from hypothesis import given, settings, strategies as st


def _check_invariants(keys, uniq, inv):
    assert uniq.dtype == np.int64 and inv.dtype == np.int32
    assert inv.shape == keys.shape
    assert np.all(uniq[1:] > uniq[:-1])                  # sorted, no duplicates
    assert set(uniq.tolist()) == set(keys.tolist())      # same key set
    if keys.size:
        assert np.array_equal(uniq[inv], keys)           # inverse maps back
    assert uniq.size <= keys.size


def test_matches_numpy_unique_on_zipf_batches(orc):
    import workloads
    for seed in range(3):
        keys = workloads.tiny(seed=seed, n=20000).keys
        u, inv = orc.dedup(keys)
        nu, ninv = np.unique(keys, return_inverse=True)
        assert np.array_equal(u, nu)
        assert np.array_equal(inv, ninv.astype(np.int32).reshape(-1))
        _check_invariants(keys, u, inv)


def test_special_cases(orc):
    u, inv = orc.dedup(np.empty(0, dtype=np.int64))
    assert u.size == 0 and inv.size == 0
    keys = np.full(1000, 42, dtype=np.int64)
    u, inv = orc.dedup(keys)
    assert u.tolist() == [42] and np.all(inv == 0)
    keys = np.random.default_rng(1).permutation(5000).astype(np.int64) * 7 - 9000
    u, inv = orc.dedup(keys)
    assert u.size == keys.size
    assert np.array_equal(np.sort(keys), u)
    # every 64-bit value is a valid dedup key, including the table's reserved ones
    ext = np.array([-1, -2, np.iinfo(np.int64).min, np.iinfo(np.int64).max, 0, -1, -2],
                   dtype=np.int64)
    u, inv = orc.dedup(ext)
    _check_invariants(ext, u, inv)
    assert u.size == 5


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(min_value=-(2**63), max_value=2**63 - 1), max_size=300),
       st.integers(min_value=0, max_value=5))
def test_property_random_lists(orc, vals, dup_factor):
    keys = np.array(vals * (1 + dup_factor), dtype=np.int64)
    np.random.default_rng(len(vals)).shuffle(keys)
    u, inv = orc.dedup(keys)
    _check_invariants(keys, u, inv)
    nu = np.unique(keys)
    assert np.array_equal(u, nu)
