"""Pins for the oracle's eviction choice (online table, least recently used).

MTGenRec (arXiv 2505.12663), Abstract: embeddings are inserted and deleted in
real time; MTGR (arXiv 2505.18654) section 5: keys carry metadata and the
table supports compact key scanning.  The pages name no eviction policy; the
reading is: evict floor(live * num / den) live keys, smallest by
(last_seen, key).  Pin: brute force against Python's sorted() over a
randomised insert/erase history, and the effect of erasing the victims.
"""
import numpy as np


def test_victims_match_sorted_model(orc):
    rng = np.random.default_rng(2)
    t = orc.Table(1 << 12, 2)
    model = {}
    for step in range(12):
        ks = rng.integers(-500, 500, 120).astype(np.int64)
        ks = ks[(ks != -1) & (ks != -2)]
        ks = np.unique(ks)
        st = t.find_or_insert(ks, step=step)
        assert np.all(st <= 1)
        for k in ks:
            model[int(k)] = step
        for num, den in ((1, 20), (1, 3), (0, 5), (7, 7)):
            want = sorted(model, key=lambda k: (model[k], k))[: len(model) * num // den]
            assert t.lru_victims(num, den).tolist() == want
        vic = t.lru_victims(1, 20)
        assert np.all(t.erase(vic) == orc.ERASED)
        for k in vic:
            del model[int(k)]
        assert len(t) == len(model)
        lk, ls = t.live()
        assert lk.tolist() == sorted(model)
        assert ls.tolist() == [model[k] for k in sorted(model)]
