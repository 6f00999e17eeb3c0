"""Pins for the oracle's dynamic table: find-or-insert, erase, rows, metadata.

MTGenRec (arXiv 2505.12663), Abstract: dynamic hash tables replace static
ones so sparse embeddings can be inserted and deleted in real time; MTGR
(arXiv 2505.18654) section 5, "Embedding Management": each key leads to its
embedding row and its metadata.  The table contract read from these: FOUND for a live
key, INSERTED (with the closed-form initial row) for a new one, FULL when all
M slots are live, RESERVED for the two key values the table keeps for itself
(-1 empty, -2 tombstone); erase gives ERASED or NOT_FOUND; FOUND and INSERTED
stamp last_seen with the call's step.

Pins: brute force over every insert/erase sequence of length <= 5 on 3 keys at
capacities 1..4 against a Python set model; the fill-to-full special case;
rows equal the closed form after insert and after erase + re-insert.
"""
import itertools

import numpy as np
import pytest


def _model_apply(live, cap, op, key):
    if op == "ins":
        if key in live:
            return 0
        if len(live) >= cap:
            return 2
        live.add(key)
        return 1
    if key in live:
        live.remove(key)
        return 1
    return 0


@pytest.mark.parametrize("cap", [1, 2, 3, 4])
def test_brute_force_sequences_against_set_model(orc, cap):
    keys = [11, -7, 1 << 50]
    ops = [(o, k) for o in ("ins", "era") for k in keys]
    for length in range(1, 6):
        for seq in itertools.product(ops, repeat=length):
            t = orc.Table(cap, 4)
            live = set()
            for op, k in seq:
                want = _model_apply(live, cap, op, k)
                got = (t.find_or_insert([k]) if op == "ins" else t.erase([k]))[0]
                assert got == want, (cap, seq)
                assert len(t) == len(live)
            lk, _ = t.live()
            assert lk.tolist() == sorted(live)


def test_reserved_keys(orc):
    t = orc.Table(16, 4)
    st = t.find_or_insert([-1, -2, 5, -1])
    assert st.tolist() == [orc.RESERVED, orc.RESERVED, orc.INSERTED, orc.RESERVED]
    assert len(t) == 1
    assert t.erase([-1, -2]).tolist() == [orc.NOT_FOUND, orc.NOT_FOUND]


@pytest.mark.parametrize("k", range(1, 7))
def test_fill_to_full_then_replay(orc, k):
    M = 1 << k
    t = orc.Table(M, 4)
    keys = np.arange(M, dtype=np.int64) * 1000 + 3
    assert np.all(t.find_or_insert(keys) == orc.INSERTED)
    assert t.find_or_insert([999_999])[0] == orc.FULL
    assert np.all(t.find_or_insert(keys) == orc.FOUND)
    # freeing one slot lets exactly one new key in
    assert t.erase(keys[:1])[0] == orc.ERASED
    assert t.find_or_insert([999_999, 888_888]).tolist() == [orc.INSERTED, orc.FULL]


def test_rows_are_closed_form_and_reset_on_reinsert(orc):
    for dtype in (orc.F32, orc.BF16):
        t = orc.Table(64, 12, dtype=dtype, seed=5, adam=(dtype == orc.F32))
        keys = np.array([3, 1 << 40, -9, 77], dtype=np.int64)
        t.find_or_insert(keys, step=4)
        for k in keys:
            row, ls, _, _ = t.lookup(k)
            assert np.array_equal(row, orc.init_row(k, 12, dtype, seed=5))
            assert ls == 4
        if dtype == orc.F32:
            t.adam(keys[:1], np.ones((1, 12), np.float32), step=1)
            assert not np.array_equal(t.lookup(3)[0], orc.init_row(3, 12, dtype, seed=5))
        t.erase(keys[:1])
        assert t.lookup(3) is None
        assert t.find_or_insert(keys[:1], step=9)[0] == orc.INSERTED
        row, ls, m, v = t.lookup(3)
        assert np.array_equal(row, orc.init_row(3, 12, dtype, seed=5)) and ls == 9
        if dtype == orc.F32:
            assert not m.any() and not v.any()


def test_last_seen_follows_found_and_inserted(orc):
    t = orc.Table(64, 2)
    t.find_or_insert([1, 2, 3], step=1)
    t.find_or_insert([2, 4], step=7)
    got = {k: t.lookup(k)[1] for k in (1, 2, 3, 4)}
    assert got == {1: 1, 2: 7, 3: 1, 4: 7}


@pytest.mark.parametrize("cap", [1, 2])
def test_growth_sequences_against_set_model(orc, cap):
    """Capacity growth (MTGR section 5) inside every sequence of length <= 5 of
    insert / erase / double-the-capacity on 3 keys: statuses follow the set
    model with the grown bound, and a live key's row and last_seen survive
    each growth unchanged."""
    keys = [11, -7, 1 << 50]
    ops = [(o, k) for o in ("ins", "era") for k in keys] + [("grow", None)]
    for length in range(1, 6):
        for seq in itertools.product(ops, repeat=length):
            t = orc.Table(cap, 4, orc.BF16)
            live, c = set(), cap
            for step, (op, k) in enumerate(seq):
                if op == "grow":
                    before = {q: t.lookup(q) for q in live}
                    c *= 2
                    t.resize(c)
                    for q, (row, ls, _, _) in before.items():
                        row2, ls2, _, _ = t.lookup(q)
                        assert np.array_equal(row, row2) and ls == ls2
                    continue
                want = _model_apply(live, c, op, k)
                got = (t.find_or_insert([k], step=step) if op == "ins" else t.erase([k]))[0]
                assert got == want, (cap, seq)
            lk, _ = t.live()
            assert lk.tolist() == sorted(live)


def test_resize_below_live_count_is_refused(orc):
    t = orc.Table(4, 4)
    t.find_or_insert([1, 2, 3])
    with pytest.raises(ValueError):
        t.resize(2)
    t.resize(3)
    assert t.find_or_insert([4])[0] == orc.FULL
