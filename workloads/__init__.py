"""Seeded synthetic input generators for the sparse-embedding lookup path.

This module only draws inputs: feature-ID streams, bag layouts, gradients and
the prefill key sets.  It holds none of the lookup method's arithmetic (no
table hashing, no row initialisation, no dedup), so both the HIP library's
tests and the CPU oracle can be fed from it without sharing any code.

The workloads stand in for the production click logs that the MTGR paper
(arXiv 2505.18654, section 6.1 "Experiment setup") trains on, which are not
public.  Shapes follow the five workload presets below:

* ``tiny``:      65,536 IDs, Zipf(a=1.1) over a 2^20 universe, dim 16 fp32.
* ``single_large_table``: 2^22 IDs, Zipf(1.05) over 2^40, a 2^24-slot table
  pre-filled with the 2^23 most popular keys, dim 64 fp32.
* ``merged_tables``: 26 feature tables with vocabularies on a log-uniform grid
  10^3..10^8, merged into one key space as ``(table_id << 48) | id``; bags of
  Poisson(20) IDs per (sample, table); 65,536 samples; dim 128 bf16.
* ``backward``:  2^23 IDs, Zipf(1.2) over 2^40, with N(0,1) fp32 gradient rows
  of dim 128.
* ``dynamic_online``: 50 steps of 2^22 IDs, Zipf(1.05) over a sliding window
  of 2^24 ids that moves by 10% of its width per step; dim 64 bf16, 2^27 slots.

Common rules:

* RNG is ``numpy.random.Generator(PCG64(seed))``.
* Zipf(a) over K is ``rng.zipf(a)`` with draws above K redrawn.
* Rank r (1-based) maps to a key through :func:`scramble`, a bijection on
  k-bit integers (odd multiplies and xor-shifts are invertible mod 2^k), so
  popular keys are spread over the key space rather than clustered at 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "scramble", "zipf_ranks", "tiny", "single_large_table", "merged_tables",
    "backward", "dynamic_online_step", "DynamicOnlineSpec", "DynamicOnlineStream", "LookupWorkload",
    "PooledWorkload", "BackwardWorkload", "merged_vocab_sizes", "WORKLOADS",
]

_M1 = np.uint64(0x9E3779B97F4A7C15)
_M2 = np.uint64(0xBF58476D1CE4E5B9)


def scramble(x, k: int) -> np.ndarray:
    """Bijection on k-bit unsigned integers (1 <= k <= 64).

    x -> x*M1 mod 2^k; x ^= x >> ceil(k/2); x -> x*M2 mod 2^k; x ^= x >> ceil(k/2).
    Used only to place Zipf ranks in the key space.
    """
    x = np.asarray(x, dtype=np.uint64).copy()
    mask = np.uint64((1 << k) - 1) if k < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    s = np.uint64((k + 1) // 2)
    with np.errstate(over="ignore"):
        x = (x * _M1) & mask
        x ^= x >> s
        x = (x * _M2) & mask
        x ^= x >> s
    return x


def zipf_ranks(rng: np.random.Generator, a: float, K: int, n: int) -> np.ndarray:
    """n Zipf(a) ranks in [1, K]: ``rng.zipf(a)`` with draws above K redrawn."""
    out = rng.zipf(a, size=n).astype(np.int64)
    bad = np.flatnonzero(out > K)
    while bad.size:
        out[bad] = rng.zipf(a, size=bad.size)
        bad = bad[out[bad] > K]
    return out


@dataclass
class LookupWorkload:
    """One forward lookup batch against a table of ``2**capacity_log2`` slots."""
    name: str
    keys: np.ndarray                 # int64 [N]
    capacity_log2: int
    dim: int
    dtype: str                       # "f32" | "bf16"
    prefill: Optional[np.ndarray] = None   # int64 keys inserted (untimed) before the batch
    meta: dict = field(default_factory=dict)


@dataclass
class PooledWorkload(LookupWorkload):
    offsets: Optional[np.ndarray] = None    # int32 [nbags + 1], CSR over keys
    nbags: int = 0


@dataclass
class BackwardWorkload(LookupWorkload):
    grad: Optional[np.ndarray] = None       # float32 [N, dim]


def tiny(seed: int = 0, n: int = 65536) -> LookupWorkload:
    """65,536 IDs ~ Zipf(1.1) over 2^20; 2^18-slot empty table; dim 16 fp32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    r = zipf_ranks(rng, 1.1, 1 << 20, n)
    keys = scramble(r - 1, 20).astype(np.int64)
    return LookupWorkload("tiny", keys, 18, 16, "f32",
                          meta={"zipf_a": 1.1, "universe_log2": 20, "seed": seed})


def single_large_table(seed: int = 0, n: int = 1 << 22, capacity_log2: int = 24,
                       prefill_count: int = 1 << 23, universe_log2: int = 40,
                       dim: int = 64) -> LookupWorkload:
    """2^22 IDs ~ Zipf(1.05) over 2^40; 2^24 slots pre-filled with the top 2^23 ranks.

    Pre-filling the most popular 2^23 ranks gives a per-draw hit rate near
    74%; the sizes are parameters so tests can run the same shape smaller.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    r = zipf_ranks(rng, 1.05, 1 << universe_log2, n)
    keys = scramble(r - 1, universe_log2).astype(np.int64)
    prefill = scramble(np.arange(prefill_count, dtype=np.uint64), universe_log2).astype(np.int64)
    return LookupWorkload("single_large_table", keys, capacity_log2, dim, "f32", prefill=prefill,
                          meta={"zipf_a": 1.05, "universe_log2": universe_log2, "seed": seed,
                                "prefill_count": prefill_count})


N_MERGED_TABLES = 26


def merged_vocab_sizes(n_tables: int = N_MERGED_TABLES) -> np.ndarray:
    """vocab_t = round(10^(3 + 5 t / (n_tables - 1))): a log-uniform grid 1e3..1e8."""
    t = np.arange(n_tables, dtype=np.float64)
    return np.rint(10.0 ** (3.0 + 5.0 * t / (n_tables - 1))).astype(np.int64)


def merged_tables(seed: int = 0, batch: int = 65536, mean_bag: float = 20.0,
                  capacity_log2: int = 26, dim: int = 128,
                  n_tables: int = N_MERGED_TABLES) -> PooledWorkload:
    """Multi-hot bags over 26 tables merged into one key space.

    Bag b = sample * n_tables + table holds Poisson(mean_bag) IDs drawn
    Zipf(1.05) over that table's vocabulary; key = (table << 48) | (rank - 1).
    Bags are laid out sample-major and described by int32 CSR offsets.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    vocab = merged_vocab_sizes(n_tables)
    lengths = rng.poisson(mean_bag, size=(batch, n_tables)).astype(np.int64)
    flat = lengths.reshape(-1)
    offsets = np.zeros(flat.size + 1, dtype=np.int64)
    np.cumsum(flat, out=offsets[1:])
    n = int(offsets[-1])
    assert n < (1 << 31)
    table_of = np.repeat(np.tile(np.arange(n_tables, dtype=np.int64), batch), flat)
    keys = np.empty(n, dtype=np.int64)
    for t in range(n_tables):
        pos = np.flatnonzero(table_of == t)
        r = zipf_ranks(rng, 1.05, int(vocab[t]), pos.size)
        keys[pos] = (np.int64(t) << np.int64(48)) | (r - 1)
    return PooledWorkload("merged_tables", keys, capacity_log2, dim, "bf16",
                          offsets=offsets.astype(np.int32), nbags=int(flat.size),
                          meta={"zipf_a": 1.05, "n_tables": n_tables, "batch": batch,
                                "mean_bag": mean_bag, "seed": seed})


def backward(seed: int = 0, n: int = 1 << 23, dim: int = 128, capacity_log2: int = 24,
             universe_log2: int = 40, with_grad: bool = True) -> BackwardWorkload:
    """2^23 IDs ~ Zipf(1.2) over 2^40 with N(0,1) fp32 gradient rows.

    The IDs come from PCG64(seed); the gradients from a second, independent
    stream PCG64(seed + 1_000_003).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    r = zipf_ranks(rng, 1.2, 1 << universe_log2, n)
    keys = scramble(r - 1, universe_log2).astype(np.int64)
    grad = None
    if with_grad:
        grng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
        grad = grng.standard_normal((n, dim), dtype=np.float32)
    return BackwardWorkload("backward", keys, capacity_log2, dim, "f32", grad=grad,
                            meta={"zipf_a": 1.2, "universe_log2": universe_log2, "seed": seed})


@dataclass
class DynamicOnlineSpec:
    """Parameters of the drifting online stream.

    At step s the active ids are [s*delta, s*delta + window) with
    delta = window // 10, so 10% of the id range is new at every step.
    Popularity among active ids follows ascending ``scramble(u, 64)``, so an
    id keeps its relative popularity while it stays active, and new ids land
    at random popularity.  Rank ~ Zipf(a) over the window picks the id; the
    key is ``scramble(u, 40)``.
    """
    window: int = 1 << 24
    n: int = 1 << 22
    steps: int = 50
    zipf_a: float = 1.05
    capacity_log2: int = 27
    dim: int = 64
    evict_num: int = 1           # evict floor(live * 1 / 20) = 5% per step
    evict_den: int = 20

    @property
    def delta(self) -> int:
        return self.window // 10


def dynamic_online_step(spec: DynamicOnlineSpec, step: int) -> np.ndarray:
    """The int64 key batch of one online step (seed = step)."""
    rng = np.random.Generator(np.random.PCG64(step))
    lo = step * spec.delta
    active = np.arange(lo, lo + spec.window, dtype=np.uint64)
    order = np.argsort(scramble(active, 64), kind="stable")
    r = zipf_ranks(rng, spec.zipf_a, spec.window, spec.n)
    ids = active[order[r - 1]]
    return scramble(ids, 40).astype(np.int64)


class DynamicOnlineStream:
    """The same key batches as :func:`dynamic_online_step`, for steps
    0..steps-1, computed from one sort of every id the stream can reach
    (scramble64 is a bijection, so the order restricted to each window is the
    window's own order)."""

    def __init__(self, spec: DynamicOnlineSpec, steps: int):
        self.spec = spec
        self.steps = steps
        span = (steps - 1) * spec.delta + spec.window
        ids = np.arange(span, dtype=np.uint64)
        # scramble is a bijection, so the sort keys are distinct and any sort
        # gives the one order (no stable sort needed)
        self._order = ids[np.argsort(scramble(ids, 64))]

    def keys(self, step: int) -> np.ndarray:
        assert 0 <= step < self.steps
        spec = self.spec
        lo = np.uint64(step * spec.delta)
        # ids below lo wrap to huge values, so one unsigned compare tests the window
        with np.errstate(over="ignore"):
            in_window = (self._order - lo) < np.uint64(spec.window)
        ordered = self._order[in_window]
        rng = np.random.Generator(np.random.PCG64(step))
        r = zipf_ranks(rng, spec.zipf_a, spec.window, spec.n)
        return scramble(ordered[r - 1], 40).astype(np.int64)


WORKLOADS = {
    "tiny": tiny,
    "single_large_table": single_large_table,
    "merged_tables": merged_tables,
    "backward": backward,
}
