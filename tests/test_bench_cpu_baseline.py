"""bench.py's CPU-baseline legs (the oracle timed beside each workload) on
tiny samples: every leg runs, reports the fields the bench line carries, and
leaves the work it times consistent (a pass's inserts are erased before the
next, so repeated passes see the same table)."""
import os
import sys

import numpy as np

import workloads

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

FIELDS = {"value", "unit", "cores", "kind", "sample", "host_cpus"}


def _check(res):
    assert FIELDS <= set(res)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["unit"] == "Mkeys/s"
    assert res["value"] > 0


def test_lookup_leg():
    w = workloads.single_large_table(n=4096, capacity_log2=14, prefill_count=2048)
    _check(bench._cpu_baseline_lookup(w, 3000, reps=2))


def test_pooled_leg():
    w = workloads.merged_tables(batch=64, capacity_log2=18, dim=16)
    warm = workloads.merged_tables(seed=1, batch=64, capacity_log2=18, dim=16)
    res = bench._cpu_baseline_pooled(w, warm, samples=32, reps=2)
    _check(res)
    assert "first 32 samples" in res["sample"]


def test_backward_leg():
    w = workloads.backward(n=4096, dim=8, capacity_log2=14, with_grad=False)
    g = np.random.default_rng(3).standard_normal((1024, 8), dtype=np.float32)
    res = bench._cpu_baseline_backward(w, g, reps=2)
    _check(res)
    assert "first 1024 IDs" in res["sample"]


def test_online_leg():
    spec = workloads.DynamicOnlineSpec(window=1 << 12, n=1 << 10, capacity_log2=14, dim=8)
    res = bench._cpu_baseline_online(workloads, spec, steps=3, m=1 << 9)
    _check(res)
    assert res["lru_choice_and_erase_ms"] >= 0


def test_traffic_records_follow_their_sources(tmp_path, monkeypatch):
    """A workload's counter record is reported while the sources it names
    hash to the recorded value, and not once any of them changes (checked on
    a temporary record over copies of the sources)."""
    import hashlib
    import shutil
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "csrc"
    src.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for name, (record, sources) in bench.TRAFFIC_RECORDS.items():
        for f in sources:
            shutil.copy(os.path.join(bench.CSRC, f), src / f)
        h = hashlib.sha256()
        for f in sources:
            h.update((src / f).read_bytes())
        (tmp_path / "profiles" / record).write_text(
            f"# test record\nsource_sha256 = {h.hexdigest()}\ntraffic_bytes_per_launch = 12345\n")
        with monkeypatch.context() as m:
            m.setattr(bench, "CSRC", str(src))
            assert bench._measured_traffic(name) == 12345, name
            for changed in sources:
                keep = (src / changed).read_bytes()
                (src / changed).write_bytes(keep + b"\n")
                assert bench._measured_traffic(name) is None, (name, changed)
                (src / changed).write_bytes(keep)
