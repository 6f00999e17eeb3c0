"""MI355X-native sparse-embedding lookup: dedup -> dynamic hash table -> gather.

Python face of libhtl.so (include/htl.h).  The library implements, as HIP
kernels for gfx950, the embedding path described by MTGenRec (arXiv
2505.12663: embeddings in a dynamic hash table, feature tables merged into
one, IDs deduplicated in two stages) and MTGR (arXiv 2505.18654, section 5): feature-ID dedup,
find-or-insert into an open-addressing table with odd-step probing, row
gather with optional bag sum-pooling, gradient segment-sum and row-wise Adam,
erase and least-recently-used eviction.

Build the library first: ``python -m hash_table_lookup_amd.build``.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._binding import (  # noqa: F401
    DEDUP_BINS_ONLY, DEDUP_DEVICE_SET, DEDUP_ONE_TILE, DEDUP_TWO_STAGE_BINS, DedupPlan,
    ADAM_STATE, BF16, EMPTY_KEY, ERASED, EXPORTED, F32, FOUND, FULL, GROWABLE, HTLError, INSERTED, LIB_PATH,
    META_ACCESS_LOG, DEBUG_DEDUP, DEBUG_DUP, DEBUG_FULL, DEBUG_LOG, DEBUG_SLOT, DEBUG_WALK, copy_probe,
    copy_to_device_ptr, debug_build, debug_flags,
    META_LAST_SEEN, NOT_FOUND, RESERVED, TOMBSTONE_KEY, Table, dedup_unique_inverse, gather,
    gather_pool, lib, lookup_fused, lookup_slots, release_workspaces, rowwise_adam, segment_sum, segment_sum_adam, table_keys,
    table_tensor,
)

from .pipeline import LookupPipeline, PipelineBatch  # noqa: F401

__all__ = [
    "Table", "DedupPlan", "LookupPipeline", "PipelineBatch", "dedup_unique_inverse", "gather", "gather_pool", "segment_sum", "rowwise_adam",
    "segment_sum_adam", "lookup", "lookup_fused", "lookup_slots", "lib", "release_workspaces", "HTLError", "FOUND", "INSERTED", "FULL", "RESERVED", "NOT_FOUND", "ERASED",
]


def lookup(table: Table, keys: torch.Tensor, step: int = 0,
           offsets: Optional[torch.Tensor] = None, out_dtype=None, fused: bool = True):
    """The forward hot path on one batch of feature IDs.

    dedup_unique_inverse -> ht_find_or_insert (absent keys inserted) ->
    emb_gather_pool.  Returns (out, unique, inverse, n_unique, slots, status);
    out is per-ID rows, or per-bag sums when CSR ``offsets`` are given.
    fused=True makes the one emb_lookup call, False the three calls.
    """
    if fused:
        od = out_dtype
        if offsets is not None and od is None:
            od = table.dtype
        return lookup_fused(table, keys, step, offsets, od)
    unique, inverse, n_unique = dedup_unique_inverse(keys)
    slots, status = table.find_or_insert(unique, n_dev=n_unique, step=step)
    if offsets is None:
        out = gather(table, slots, inverse, out_dtype=out_dtype)
    else:
        out = gather_pool(table, slots, inverse, offsets,
                          out_dtype=out_dtype if out_dtype is not None else table.dtype)
    return out, unique, inverse, n_unique, slots, status
