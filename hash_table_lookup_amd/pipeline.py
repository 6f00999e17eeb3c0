"""Copy / lookup / compute overlap for batches that arrive in host memory.

MTGR (arXiv 2505.18654) section 5, "Other Optimizations": three streams run
at once -- one copies the next batch from the CPU to the GPU, one looks up
the embeddings of the current batch, one computes the model on the batch
before.  LookupPipeline is that arrangement for this library's lookup:

* a copy stream moves batch i+1's keys from pinned host memory into a
  device key buffer while
* the lookup stream runs batch i's lookup (emb_lookup_slots and the gather,
  or bag pooling) into an output buffer, while
* the caller's own (compute) stream consumes batch i-1's rows.

Buffers rotate over `depth` slots (default 2).  Events order the streams:
the lookup of a batch waits for its copy; the copy into a key buffer waits
for the lookup that last read it; the lookup into an output slot waits for
the caller to have finished with that slot's previous batch, which the
pipeline records on the caller's current stream when the caller asks for
the next batch.  Every stream keeps the default priority.

The library's calls only enqueue work on the stream they are given, so
this class is stream plumbing around them (torch supplies the streams,
events and memory); every step of the lookup runs in the library's kernels.
"""
from __future__ import annotations

from typing import Iterable, Iterator, NamedTuple

import numpy as np
import torch

from . import _binding as B


class PipelineBatch(NamedTuple):
    """One looked-up batch.  Its tensors are ready once the caller's stream
    has waited on `ready` (done for the caller's current stream before the
    batch is handed out); they stay valid until the caller asks for batch
    index + depth."""
    index: int
    out: torch.Tensor          # [n, dim] rows, or [nbags, dim] bag sums
    unique: torch.Tensor
    inverse: torch.Tensor
    n_unique: torch.Tensor
    slots: torch.Tensor
    status: torch.Tensor
    ready: torch.cuda.Event


class LookupPipeline:
    """Overlaps the host-to-device copy of the next batch with the lookup of
    the current one and the caller's use of the previous one."""

    def __init__(self, table: B.Table, n_max: int, depth: int = 2, out_dtype=None, nbags_max: int = 0):
        if depth < 2:
            raise ValueError("depth must be at least 2")
        dev = table.device
        self.table, self.n_max, self.depth = table, n_max, depth
        self.od = table.dtype if out_dtype is None else B._dtype_code(out_dtype)
        self.copy_stream = torch.cuda.Stream(device=dev)      # default priority
        self.lookup_stream = torch.cuda.Stream(device=dev)    # default priority
        self.host = [torch.empty(n_max, dtype=torch.int64, pin_memory=True) for _ in range(depth)]
        self.keys = [torch.empty(n_max, dtype=torch.int64, device=dev) for _ in range(depth)]
        rows = max(n_max, nbags_max)
        odt = B._TORCH_DTYPE[self.od]
        self.outs = [torch.empty((rows, table.dim), dtype=odt, device=dev) for _ in range(depth)]
        self.bufs = [{"unique": torch.empty(max(n_max, 1), dtype=torch.int64, device=dev),
                      "inverse": torch.empty(max(n_max, 1), dtype=torch.int32, device=dev),
                      "n_unique": torch.empty(1, dtype=torch.int64, device=dev),
                      "slots": torch.empty(max(n_max, 1), dtype=torch.int32, device=dev),
                      "status": torch.empty(max(n_max, 1), dtype=torch.uint8, device=dev),
                      "id_slots": torch.empty(max(n_max, 1), dtype=torch.int32, device=dev)}
                     for _ in range(depth)]
        self.copied = [torch.cuda.Event() for _ in range(depth)]      # keys of slot s are on the device
        self.keys_free = [None] * depth                               # lookup done reading keys of slot s
        self.out_free = [None] * depth                                # caller done with outputs of slot s

    def _copy(self, i: int, batch) -> int:
        s = i % self.depth
        keys = batch[0] if isinstance(batch, tuple) else batch
        n = int(keys.shape[0])
        if n > self.n_max:
            raise ValueError(f"batch {i} holds {n} keys, more than n_max = {self.n_max}")
        src = torch.from_numpy(np.ascontiguousarray(keys, dtype=np.int64)) if isinstance(keys, np.ndarray) else keys
        self.copied[s].synchronize()                     # the last copy out of this pinned buffer has left
        self.host[s][:n].copy_(src)                      # into pinned memory (host side)
        with torch.cuda.stream(self.copy_stream):
            if self.keys_free[s] is not None:
                self.copy_stream.wait_event(self.keys_free[s])
            self.keys[s][:n].copy_(self.host[s][:n], non_blocking=True)
            self.copied[s].record(self.copy_stream)
        return n

    def _lookup(self, idx: int, n: int, offsets, step: int):
        s = idx % self.depth
        with torch.cuda.stream(self.lookup_stream):
            self.lookup_stream.wait_event(self.copied[s])
            if self.out_free[s] is not None:
                self.lookup_stream.wait_event(self.out_free[s])
            b = self.bufs[s]
            uniq, inv, nu, slots, status, ids = B.lookup_slots(
                self.table, self.keys[s][:n], step=step,
                bufs={k: (v[:n] if k != "n_unique" else v) for k, v in b.items()})
            kf = torch.cuda.Event()
            kf.record(self.lookup_stream)            # the dedup has read the keys of slot s
            if offsets is None:
                out = B.gather(self.table, ids, None, out=self.outs[s][:n])
            else:
                out = B.gather_pool(self.table, ids, None, offsets, out_dtype=self.od,
                                    out=self.outs[s][:offsets.numel() - 1])
            ready = torch.cuda.Event()
            ready.record(self.lookup_stream)
        self.keys_free[s] = kf
        return PipelineBatch(idx, out, uniq, inv, nu, slots, status, ready)

    def run(self, batches: Iterable, step0: int = 0, steps_per_batch: int = 1) -> Iterator[PipelineBatch]:
        """Looks up every batch (a numpy / CPU int64 key array, or a tuple
        (keys, offsets) with int32 device CSR offsets for bag sums) and
        yields them in order; batch i is stamped with step step0 + i *
        steps_per_batch.  While the caller works on batch i (on its current
        stream), batch i+1 is being looked up and batch i+2 copied."""
        it = iter(batches)
        copied = []          # (index, n, offsets): on the device or on their way, not looked up
        count = 0

        def feed():
            nonlocal count
            try:
                b = next(it)
            except StopIteration:
                return
            n = self._copy(count, b)
            copied.append((count, n, b[1] if isinstance(b, tuple) else None))
            count += 1

        feed()
        feed()
        ahead = None
        if copied:
            idx, n, off = copied.pop(0)
            ahead = self._lookup(idx, n, off, step0 + idx * steps_per_batch)
        while ahead is not None:
            cur = ahead
            ahead = None
            if copied:                                    # the next lookup, one batch ahead
                idx, n, off = copied.pop(0)
                ahead = self._lookup(idx, n, off, step0 + idx * steps_per_batch)
            feed()                                        # and the copy after it
            torch.cuda.current_stream().wait_event(cur.ready)
            yield cur
            # the caller asks for the next batch: its work on this slot is enqueued
            done = torch.cuda.Event()
            done.record(torch.cuda.current_stream())
            self.out_free[cur.index % self.depth] = done
