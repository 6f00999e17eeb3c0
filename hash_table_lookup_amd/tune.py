"""Dedup crossover sweep: times each second-stage form of the dedup on this
GPU across batch sizes and duplicate patterns, the measurement behind the
adaptive dedup's rule (skip stage 1 only while the duplicate share d that
stage 1 measured bounds the hottest key so that it cannot overfill a bin:
d * n + ntiles <= 3 n / P for P bins; the sweep shows the skip saving up
to 15% where tiles hold almost no duplicates and costing 3-14x under skew).

    python -m hash_table_lookup_amd.tune [--reps 10] [--max-log2 23]

Prints one markdown table: batch size, pattern, the share of keys that
survive stage 1 (per-tile distinct keys / n) and the share that is unique
(U / n), and the median event-timed duration of dedup_unique_inverse with
the second stage forced to each form (HTL_DEDUP_PATH).  The keys are
synthetic and seeded; only the library's kernels are timed.
"""
from __future__ import annotations

import argparse
import os

import numpy as np
import torch

from . import _binding as B

FORMS = ("bins", "bins_only", "set")


def _patterns(n: int, rng: np.random.Generator):
    """(name, keys) with duplicate shares from none to most."""
    yield "distinct", rng.choice(1 << 60, n, replace=False).astype(np.int64)
    yield "uniform 16n", rng.integers(0, 16 * n, n).astype(np.int64)
    yield "uniform 2n", rng.integers(0, 2 * n, n).astype(np.int64)
    yield "pairs", np.repeat(rng.choice(1 << 60, (n + 1) // 2, replace=False).astype(np.int64), 2)[:n]
    for a in (1.05, 1.2):
        r = rng.zipf(a, n).astype(np.uint64)
        with np.errstate(over="ignore"):        # an odd multiply spreads the ranks over 61 bits
            yield f"zipf {a}", ((r * np.uint64(0x9E3779B97F4A7C15)) >> np.uint64(3)).astype(np.int64)


def _survivors(keys: np.ndarray, tile: int = 2048) -> int:
    return sum(np.unique(keys[b:b + tile]).size for b in range(0, keys.size, tile))


def _time(keys: torch.Tensor, reps: int) -> float:
    stream = torch.cuda.current_stream()
    B.dedup_unique_inverse(keys)                 # warm-up (workspace, code)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        B.dedup_unique_inverse(keys)
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return float(np.median(ts))


def sweep(reps: int = 10, max_log2: int = 23):
    rng = np.random.default_rng(2025)
    rows = []
    saved = os.environ.get("HTL_DEDUP_PATH")
    try:
        for lg in [g for g in (14, 16, 18, 20, 22, 23) if g <= max_log2]:
            n = 1 << lg
            for name, keys_np in _patterns(n, rng):
                keys = torch.from_numpy(keys_np).cuda()
                us = {}
                for form in FORMS:
                    os.environ["HTL_DEDUP_PATH"] = form
                    us[form] = _time(keys, reps)
                rows.append((lg, name, _survivors(keys_np) / n, np.unique(keys_np).size / n, us))
                print(f"2^{lg} {name}: " + ", ".join(f"{k} {v:.1f} us" for k, v in us.items()), flush=True)
    finally:
        if saved is None:
            os.environ.pop("HTL_DEDUP_PATH", None)
        else:
            os.environ["HTL_DEDUP_PATH"] = saved
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--max-log2", type=int, default=23)
    a = ap.parse_args()
    rows = sweep(a.reps, a.max_log2)
    print("\n| n | keys | survive stage 1 | unique | two-stage bins (us) | bins, no stage 1 (us) | device set (us) |")
    print("|---|---|---|---|---|---|---|")
    for lg, name, s, u, us in rows:
        best = min(us, key=us.get)
        cells = [f"**{us[f]:.1f}**" if f == best else f"{us[f]:.1f}" for f in FORMS]
        print(f"| 2^{lg} | {name} | {s:.3f} | {u:.3f} | " + " | ".join(cells) + " |")


if __name__ == "__main__":
    main()
