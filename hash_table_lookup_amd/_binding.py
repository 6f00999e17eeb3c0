"""ctypes binding of libhtl.so: argument marshalling only.

Every step of the lookup path runs in the library's HIP kernels; this module
checks tensor dtypes/devices, allocates outputs and workspaces with torch
(device memory and streams are all torch is used for), and passes raw device
pointers plus the current HIP stream through the C ABI declared in
include/htl.h.  There is no CPU fallback: if the library is missing, or no
GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# HTL_LIB names another build of the library (the sanitizer build, say)
LIB_PATH = os.environ.get("HTL_LIB") or os.path.join(_HERE, "libhtl.so")

HTL_OK, HTL_ERR_INVALID, HTL_ERR_NOMEM, HTL_ERR_DEVICE = 0, 1, 2, 3
F32, BF16 = 0, 1
FOUND, INSERTED, FULL, RESERVED = 0, 1, 2, 3
NOT_FOUND, ERASED = 0, 1
META_LAST_SEEN, ADAM_STATE, GROWABLE, META_ACCESS_LOG = 1, 2, 4, 8
EMPTY_KEY, TOMBSTONE_KEY = -1, -2

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_I32 = ctypes.c_int
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_F = ctypes.c_float


class HTLError(RuntimeError):
    """A libhtl call returned an error status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libhtl error {status}: {message}")
        self.status = status


class _View(ctypes.Structure):
    _fields_ = [("capacity", _I64), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("keys", _P), ("rows", _P), ("last_seen", _P), ("adam_m", _P), ("adam_v", _P),
                ("row_of_slot", _P)]


_SIGNATURES = {
    "ht_create": [ctypes.POINTER(_P), _I32, _I32, _I32, _U64, _U32, _P],
    "ht_destroy": [_P],
    "ht_clear": [_P, _P],
    "ht_resize": [_P, _I32, _P],
    "ht_find_or_insert": [_P, _P, _I64, _P, _U32, _P, _P, _P],
    "ht_erase": [_P, _P, _I64, _P, _P],
    "ht_scan": [_P, _P, _P, _P, _P, _P],
    "ht_export": [_P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P],
    "ht_import": [_P, _P, _I64, _P, _P, _P, _P, _P, _P],
    "lru_workspace_bytes": [_P],
    "ht_lru_select": [_P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P],
    "ht_rows": [_P, ctypes.POINTER(_P), ctypes.POINTER(_I64)],
    "ht_access_log_state": [_P, _P, _P],
    "ht_access_log_rebuild": [_P, _P],
    "htl_debug_build": [],
    "htl_debug_flags": [ctypes.POINTER(_U32)],
    "ht_view": [_P, ctypes.POINTER(_View)],
    "dedup_workspace_bytes": [_I64],
    "dedup_unique_inverse": [_P, _I64, _P, _P, _P, _P, _SZ, _P],
    "dedup_unique_inverse_ordered": [_P, _I64, _P, _P, _P, _P, _SZ, _P],
    "dedup_plan_create": [ctypes.POINTER(_P)],
    "dedup_plan_destroy": [_P],
    "dedup_plan_stats": [_P, _P],
    "dedup_plan_choose": [_P, _I64],
    "dedup_unique_inverse_adaptive": [_P, _P, _I64, _P, _P, _P, _P, _SZ, _P],
    "dedup_noalloc_max_keys": [],
    "dedup_unique_inverse_noalloc": [_P, _I64, _P, _P, _P, _P],
    "emb_gather_pool": [_P, _P, _P, _I64, _P, _I64, _I32, _P, _P],
    "emb_lookup_slots": [_P, _P, _I64, _U32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "emb_lookup_workspace_bytes": [_I64],
    "emb_lookup": [_P, _P, _I64, _U32, _P, _P, _P, _P, _P, _P, _I64, _I32, _P, _P, _SZ, _P],
    "segsum_workspace_bytes": [_I64, _I64, _I32],
    "emb_grad_segment_sum": [_P, _P, _I64, _P, _I64, _I32, _P, _P, _SZ, _P],
    "emb_rowwise_adam": [_P, _P, _P, _I64, _P, _F, _F, _F, _F, _I64, _P],
    "segsum_adam_workspace_bytes": [_I64, _I64, _I32],
    "emb_grad_segment_sum_adam": [_P, _P, _P, _P, _I64, _P, _I64, _F, _F, _F, _F, _I64, _P, _SZ, _P],
    "htl_copy_probe": [_P, _P, _I64, _P],
    "htl_last_error": [],
}
_SIZE_FUNCS = {"lru_workspace_bytes", "dedup_workspace_bytes", "segsum_workspace_bytes",
               "segsum_adam_workspace_bytes", "emb_lookup_workspace_bytes"}
EXPORTED = tuple(_SIGNATURES)

_lib = None


def lib() -> ctypes.CDLL:
    """Load libhtl.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hash_table_lookup_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            if name in _SIZE_FUNCS:
                f.restype = _SZ
            elif name == "dedup_noalloc_max_keys":
                f.restype = _I64
            elif name == "dedup_plan_choose":
                f.restype = ctypes.c_int32
            elif name == "htl_last_error":
                f.restype = ctypes.c_char_p
            else:
                f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != HTL_OK:
        msg = lib().htl_last_error()
        raise HTLError(status, msg.decode() if msg else "")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.contiguous()


_ws_cache = {}


def _workspace(tag: str, nbytes: int, device) -> torch.Tensor:
    """A cached uint8 device buffer of at least nbytes (256-byte aligned by torch).

    One buffer per (path, device, stream): calls enqueued on one stream run in
    order, so they may share it; calls on two streams get two buffers and do
    not race.  A buffer that has to grow is replaced on the stream that uses
    it -- torch's allocator hands freed memory out again only in that
    stream's order -- so no work still queued reads a freed buffer."""
    key = (tag, str(device), _stream())
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def copy_probe(src: torch.Tensor, dst: torch.Tensor):
    """dst <- src with the library's streaming-copy probe kernel (a bandwidth
    reference; both contiguous, same byte size, a multiple of 16 bytes)."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("copy_probe needs contiguous GPU tensors")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("copy_probe: src and dst differ in size")
    _check(lib().htl_copy_probe(_ptr(src), _ptr(dst), nb, _stream()))


def release_workspaces() -> None:
    """Drop the cached workspaces (the next call on each path allocates anew)."""
    _ws_cache.clear()


def _dtype_code(dtype) -> int:
    if dtype in ("f32", "fp32", "float32", torch.float32, F32):
        return F32
    if dtype in ("bf16", "bfloat16", torch.bfloat16, BF16):
        return BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


class Table:
    """A dynamic embedding table living in device memory (libhtl's ht_* calls).

    growable=True: rows live apart from the key index, slots returned are row
    handles, and resize() grows the index without moving rows.
    access_log=True (with last_seen): the table keeps an access log that
    lets lru_select read only the oldest steps' entries."""

    def __init__(self, capacity_log2: int, dim: int, dtype="f32", init_seed: int = 0,
                 last_seen: bool = False, adam: bool = False, growable: bool = False,
                 access_log: bool = False):
        L = lib()
        self.capacity_log2, self.dim = capacity_log2, dim
        self.dtype = _dtype_code(dtype)
        self.init_seed = init_seed
        self.growable = growable
        flags = ((META_LAST_SEEN if last_seen else 0) | (ADAM_STATE if adam else 0)
                 | (GROWABLE if growable else 0) | (META_ACCESS_LOG if access_log else 0))
        h = _P()
        _check(L.ht_create(ctypes.byref(h), capacity_log2, dim, self.dtype,
                           init_seed & 0xFFFFFFFFFFFFFFFF, flags, _stream()))
        self._h = h
        self.device = torch.device("cuda", torch.cuda.current_device())

    @property
    def handle(self):
        return self._h

    @property
    def capacity(self) -> int:
        return 1 << self.capacity_log2

    @property
    def row_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    def close(self):
        if getattr(self, "_h", None):
            _check(lib().ht_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def clear(self):
        _check(lib().ht_clear(self._h, _stream()))

    def resize(self, capacity_log2: int):
        """Grow a growable table to 2^capacity_log2 slots (rows stay in place)."""
        _check(lib().ht_resize(self._h, capacity_log2, _stream()))
        self.capacity_log2 = capacity_log2

    def find_or_insert(self, keys: torch.Tensor, n_dev: Optional[torch.Tensor] = None,
                       step: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
        keys = _dev(keys, torch.int64, "keys")
        n = keys.numel()
        slots = torch.empty(n, dtype=torch.int32, device=keys.device)
        status = torch.empty(n, dtype=torch.uint8, device=keys.device)
        if n_dev is not None:
            n_dev = _dev(n_dev, torch.int64, "n_dev")
        _check(lib().ht_find_or_insert(self._h, _ptr(keys), n, _ptr(n_dev), step, _ptr(slots),
                                       _ptr(status), _stream()))
        return slots, status

    def erase(self, keys: torch.Tensor) -> torch.Tensor:
        keys = _dev(keys, torch.int64, "keys")
        status = torch.empty(keys.numel(), dtype=torch.uint8, device=keys.device)
        _check(lib().ht_erase(self._h, _ptr(keys), keys.numel(), _ptr(status), _stream()))
        return status

    def scan(self):
        """(keys, last_seen, slots, n_live) -- first n_live entries are valid."""
        M = self.capacity
        keys = torch.empty(M, dtype=torch.int64, device=self.device)
        ls = torch.empty(M, dtype=torch.int32, device=self.device)
        slots = torch.empty(M, dtype=torch.int32, device=self.device)
        n = torch.empty(1, dtype=torch.int64, device=self.device)
        _check(lib().ht_scan(self._h, _ptr(keys), _ptr(ls), _ptr(slots), _ptr(n), _stream()))
        return keys, ls, slots, n

    def export_buffers(self, entries: int):
        """Device buffers for an export of up to `entries` live entries."""
        cap = max(entries, 1)
        d = {"keys": torch.empty(cap, dtype=torch.int64, device=self.device),
             "rows": torch.empty((cap, self.dim), dtype=self.row_dtype, device=self.device)}
        v = self.view()
        if v.last_seen:
            d["last_seen"] = torch.empty(cap, dtype=torch.int32, device=self.device)
        if v.adam_m:
            d["adam_m"] = torch.empty((cap, self.dim), dtype=torch.float32, device=self.device)
            d["adam_v"] = torch.empty((cap, self.dim), dtype=torch.float32, device=self.device)
        d["n"] = torch.empty(1, dtype=torch.int64, device=self.device)
        return d

    def export(self, begin: int = 0, end: Optional[int] = None, bufs=None):
        """Live entries of slots [begin, end) in slot order: dict of tensors
        (keys, rows, last_seen / adam_m / adam_v when kept) and n (device int64).
        bufs: buffers from export_buffers(>= end - begin) to reuse."""
        end = self.capacity if end is None else end
        d = dict(bufs) if bufs is not None else self.export_buffers(end - begin)
        if d["keys"].numel() < end - begin:
            raise ValueError("export buffers are smaller than the slot range")
        n = d["n"]
        _check(lib().ht_export(self._h, begin, end, _ptr(d["keys"]), _ptr(d["rows"]), _ptr(d.get("last_seen")),
                               _ptr(d.get("adam_m")), _ptr(d.get("adam_v")), _ptr(n), _stream()))
        d["n"] = n
        return d

    def import_(self, keys: torch.Tensor, rows: torch.Tensor, last_seen=None, adam_m=None, adam_v=None):
        """Insert keys with the given rows (and metadata); returns the status per key."""
        keys = _dev(keys, torch.int64, "keys")
        rows = _dev(rows, self.row_dtype, "rows")
        if last_seen is not None:
            last_seen = _dev(last_seen, torch.int32, "last_seen")
        if adam_m is not None:
            adam_m = _dev(adam_m, torch.float32, "adam_m")
            adam_v = _dev(adam_v, torch.float32, "adam_v")
        status = torch.empty(keys.numel(), dtype=torch.uint8, device=keys.device)
        _check(lib().ht_import(self._h, _ptr(keys), keys.numel(), _ptr(rows), _ptr(last_seen), _ptr(adam_m),
                               _ptr(adam_v), _ptr(status), _stream()))
        return status

    def checkpoint(self, chunk_slots: int = 1 << 24):
        """The whole live state as host numpy arrays, exported range by range
        (device buffers of chunk_slots entries)."""
        parts = {}
        for b in range(0, self.capacity, chunk_slots):
            d = self.export(b, min(b + chunk_slots, self.capacity))
            n = int(d.pop("n").item())
            for name, t in d.items():
                t = t[:n]
                if t.dtype == torch.bfloat16:           # bf16 rows travel as their bits
                    t = t.view(torch.int16)
                parts.setdefault(name, []).append(t.cpu().numpy())
        return {name: np.concatenate(v) for name, v in parts.items()}

    def restore(self, ck, chunk: int = 1 << 24):
        """Import a checkpoint() (in chunks of `chunk` keys); returns the statuses."""
        out = []
        n = ck["keys"].shape[0]

        def part(name, b, e):
            if name not in ck:
                return None
            return torch.from_numpy(np.ascontiguousarray(ck[name][b:e])).to(self.device)

        for b in range(0, n, chunk):
            e = min(b + chunk, n)
            rows = part("rows", b, e)
            if self.dtype == BF16:
                rows = rows.view(torch.bfloat16)
            out.append(self.import_(part("keys", b, e), rows, part("last_seen", b, e),
                                    part("adam_m", b, e), part("adam_v", b, e)))
        return torch.cat(out) if out else torch.empty(0, dtype=torch.uint8, device=self.device)

    def lru_select(self, num: int, den: int, victims_cap: Optional[int] = None):
        """(victims, n_victims): the floor(live*num/den) least recently used keys."""
        cap = self.capacity if victims_cap is None else victims_cap
        victims = torch.empty(max(cap, 1), dtype=torch.int64, device=self.device)
        n = torch.empty(1, dtype=torch.int64, device=self.device)
        nb = lib().lru_workspace_bytes(self._h)
        ws = _workspace("lru", nb, self.device)
        _check(lib().ht_lru_select(self._h, num, den, _ptr(victims), cap, _ptr(n), _ptr(ws), nb,
                                   _stream()))
        return victims, n

    def access_log_state(self) -> torch.Tensor:
        """int64[4] on the device (ht_access_log_state): whether the log
        serves the next lru_select (1 / 0), its head, its tail, and the
        oldest step that may still have live keys."""
        out = torch.empty(4, dtype=torch.int64, device=self.device)
        _check(lib().ht_access_log_state(self._h, _ptr(out), _stream()))
        return out

    def rebuild_access_log(self):
        """ht_access_log_rebuild: the log again from the live keys (synchronises)."""
        _check(lib().ht_access_log_rebuild(self._h, _stream()))

    def rows_view(self):
        """(device address of the rows, bytes per row): the read-only row view
        of ht_rows (rows indexed by slot, or by row handle when growable)."""
        p, rb = _P(), _I64()
        _check(lib().ht_rows(self._h, ctypes.byref(p), ctypes.byref(rb)))
        return p.value, rb.value

    def view(self) -> _View:
        v = _View()
        _check(lib().ht_view(self._h, ctypes.byref(v)))
        return v


DEDUP_ONE_TILE, DEDUP_TWO_STAGE_BINS, DEDUP_BINS_ONLY, DEDUP_DEVICE_SET = 0, 1, 2, 3


class _DedupStats(ctypes.Structure):
    _fields_ = [("calls", _I64), ("n", _I64), ("survivors", _I64), ("n_unique", _I64), ("path", ctypes.c_int32)]


class DedupPlan:
    """State of the adaptive dedup (dedup_plan_*): the statistics of its
    previous calls, which pick the second-stage form of the next."""

    def __init__(self):
        h = _P()
        _check(lib().dedup_plan_create(ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            _check(lib().dedup_plan_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stats(self) -> dict:
        v = _DedupStats()
        _check(lib().dedup_plan_stats(self._h, ctypes.byref(v)))
        return {"calls": v.calls, "n": v.n, "survivors": v.survivors, "n_unique": v.n_unique, "path": v.path}

    def choose(self, n: int) -> int:
        return int(lib().dedup_plan_choose(self._h, n))

    def dedup(self, keys: torch.Tensor):
        """(unique, inverse, n_unique) as dedup_unique_inverse, adaptively."""
        keys = _dev(keys, torch.int64, "keys")
        n = keys.numel()
        unique = torch.empty(max(n, 1), dtype=torch.int64, device=keys.device)
        inverse = torch.empty(n, dtype=torch.int32, device=keys.device)
        n_unique = torch.empty(1, dtype=torch.int64, device=keys.device)
        nb = lib().dedup_workspace_bytes(n)
        ws = _workspace("dedup", nb, keys.device)
        _check(lib().dedup_unique_inverse_adaptive(self._h, _ptr(keys), n, _ptr(unique), _ptr(inverse),
                                                   _ptr(n_unique), _ptr(ws), nb, _stream()))
        return unique, inverse, n_unique


def dedup_unique_inverse(keys: torch.Tensor, ordered: bool = False):
    """(unique int64[n], inverse int32[n], n_unique int64[1]) -- unique[:U] valid.

    ordered=True lists unique keys in order of first occurrence (reproducible)."""
    keys = _dev(keys, torch.int64, "keys")
    n = keys.numel()
    unique = torch.empty(max(n, 1), dtype=torch.int64, device=keys.device)
    inverse = torch.empty(n, dtype=torch.int32, device=keys.device)
    n_unique = torch.empty(1, dtype=torch.int64, device=keys.device)
    nb = lib().dedup_workspace_bytes(n)
    ws = _workspace("dedup", nb, keys.device)
    fn = lib().dedup_unique_inverse_ordered if ordered else lib().dedup_unique_inverse
    _check(fn(_ptr(keys), n, _ptr(unique), _ptr(inverse), _ptr(n_unique), _ptr(ws), nb, _stream()))
    return unique, inverse, n_unique


def lookup_fused(table: Table, keys: torch.Tensor, step: int = 0, offsets: Optional[torch.Tensor] = None,
                 out_dtype=None, out: Optional[torch.Tensor] = None, bufs: Optional[dict] = None):
    """The forward path in one call (emb_lookup): dedup -> find-or-insert ->
    gather, or bag sums with CSR ``offsets``.  Returns (out, unique, inverse,
    n_unique, slots, status) as the three calls do.  ``bufs`` may hold
    preallocated unique / inverse / n_unique / slots / status tensors."""
    keys = _dev(keys, torch.int64, "keys")
    n = keys.numel()
    d = keys.device
    b = bufs or {}
    unique = b.get("unique")
    unique = unique if unique is not None else torch.empty(max(n, 1), dtype=torch.int64, device=d)
    inverse = b.get("inverse")
    inverse = inverse if inverse is not None else torch.empty(n, dtype=torch.int32, device=d)
    n_unique = b.get("n_unique")
    n_unique = n_unique if n_unique is not None else torch.empty(1, dtype=torch.int64, device=d)
    slots = b.get("slots")
    slots = slots if slots is not None else torch.empty(max(n, 1), dtype=torch.int32, device=d)
    status = b.get("status")
    status = status if status is not None else torch.empty(max(n, 1), dtype=torch.uint8, device=d)
    if offsets is None:
        od = table.dtype if out_dtype is None else _dtype_code(out_dtype)
        nb = 0
        shape = (n, table.dim)
    else:
        offsets = _dev(offsets, torch.int32, "offsets")
        od = table.dtype if out_dtype is None else _dtype_code(out_dtype)
        nb = offsets.numel() - 1
        shape = (nb, table.dim)
    if out is None:
        out = torch.empty(shape, dtype=_TORCH_DTYPE[od], device=d)
    nbytes = lib().emb_lookup_workspace_bytes(n)
    ws = _workspace("lookup", nbytes, d)
    _check(lib().emb_lookup(table.handle, _ptr(keys), n, step, _ptr(unique), _ptr(inverse), _ptr(n_unique),
                            _ptr(slots), _ptr(status), _ptr(offsets), nb, od, _ptr(out), _ptr(ws), nbytes,
                            _stream()))
    return out, unique, inverse, n_unique, slots, status


def lookup_slots(table: Table, keys: torch.Tensor, step: int = 0, bufs: Optional[dict] = None):
    """dedup -> find-or-insert, and each ID's slot (emb_lookup_slots).
    Returns (unique, inverse, n_unique, slots, status, id_slots); a gather of
    id_slots with no inverse gives the batch's rows."""
    keys = _dev(keys, torch.int64, "keys")
    n = keys.numel()
    d = keys.device
    b = bufs or {}

    def buf(name, size, dtype):
        t = b.get(name)
        return t if t is not None else torch.empty(size, dtype=dtype, device=d)

    unique = buf("unique", max(n, 1), torch.int64)
    inverse = buf("inverse", n, torch.int32)
    n_unique = buf("n_unique", 1, torch.int64)
    slots = buf("slots", max(n, 1), torch.int32)
    status = buf("status", max(n, 1), torch.uint8)
    id_slots = buf("id_slots", max(n, 1), torch.int32)
    nbytes = lib().dedup_workspace_bytes(n)
    ws = _workspace("dedup", nbytes, d)
    _check(lib().emb_lookup_slots(table.handle, _ptr(keys), n, step, _ptr(unique), _ptr(inverse), _ptr(n_unique),
                                  _ptr(slots), _ptr(status), _ptr(id_slots), _ptr(ws), nbytes, _stream()))
    return unique, inverse, n_unique, slots, status, id_slots


def gather(table: Table, slots: torch.Tensor, inverse: Optional[torch.Tensor] = None,
           out_dtype=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-ID rows: out[i] = rows[slots[inverse[i]]] (inverse None: identity)."""
    slots = _dev(slots, torch.int32, "slots")
    n = slots.numel() if inverse is None else inverse.numel()
    if inverse is not None:
        inverse = _dev(inverse, torch.int32, "inverse")
    od = table.dtype if out_dtype is None else _dtype_code(out_dtype)
    if out is None:
        out = torch.empty((n, table.dim), dtype=_TORCH_DTYPE[od], device=slots.device)
    _check(lib().emb_gather_pool(table.handle, _ptr(slots), _ptr(inverse), n, None, 0, od,
                                 _ptr(out), _stream()))
    return out


def gather_pool(table: Table, slots: torch.Tensor, inverse: Optional[torch.Tensor],
                offsets: torch.Tensor, out_dtype="f32", out: Optional[torch.Tensor] = None):
    """Bag sums: out[b] = sum of rows of IDs offsets[b]..offsets[b+1]-1.

    The kernels clamp every bag to [0, n), so offsets that break the CSR
    rules read no ID outside the batch; they are not checked on the host
    (reading offsets[-1] back would synchronise every call)."""
    slots = _dev(slots, torch.int32, "slots")
    offsets = _dev(offsets, torch.int32, "offsets")
    n = slots.numel() if inverse is None else inverse.numel()
    if inverse is not None:
        inverse = _dev(inverse, torch.int32, "inverse")
    nb = offsets.numel() - 1
    od = _dtype_code(out_dtype)
    if out is None:
        out = torch.empty((nb, table.dim), dtype=_TORCH_DTYPE[od], device=offsets.device)
    _check(lib().emb_gather_pool(table.handle, _ptr(slots), _ptr(inverse), n, _ptr(offsets), nb,
                                 od, _ptr(out), _stream()))
    return out


def segment_sum(grad: torch.Tensor, inverse: torch.Tensor, n_unique: Optional[torch.Tensor],
                u_max: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[u] = sum of grad[i] over inverse[i] == u, for u < n_unique (fp32)."""
    grad = _dev(grad, torch.float32, "grad")
    inverse = _dev(inverse, torch.int32, "inverse")
    n, dim = grad.shape
    if n_unique is not None:
        n_unique = _dev(n_unique, torch.int64, "n_unique")
    if out is None:
        out = torch.empty((max(u_max, 1), dim), dtype=torch.float32, device=grad.device)
    nb = lib().segsum_workspace_bytes(n, u_max, dim)
    ws = _workspace("segsum", nb, grad.device)
    _check(lib().emb_grad_segment_sum(_ptr(grad), _ptr(inverse), n, _ptr(n_unique), u_max, dim,
                                      _ptr(out), _ptr(ws), nb, _stream()))
    return out


def rowwise_adam(table: Table, slots: torch.Tensor, g: torch.Tensor,
                 n_unique: Optional[torch.Tensor], lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, step=1):
    slots = _dev(slots, torch.int32, "slots")
    g = _dev(g, torch.float32, "g")
    if n_unique is not None:
        n_unique = _dev(n_unique, torch.int64, "n_unique")
    _check(lib().emb_rowwise_adam(table.handle, _ptr(slots), _ptr(g), slots.numel(),
                                  _ptr(n_unique), lr, b1, b2, eps, step, _stream()))


def segment_sum_adam(table: Table, slots: torch.Tensor, grad: torch.Tensor, inverse: torch.Tensor,
                     n_unique: Optional[torch.Tensor], u_max: int, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8,
                     step=1):
    """Segment-sum of grad by inverse, then Adam on each unique key's table row,
    without writing the summed gradients (emb_grad_segment_sum_adam)."""
    slots = _dev(slots, torch.int32, "slots")
    grad = _dev(grad, torch.float32, "grad")
    inverse = _dev(inverse, torch.int32, "inverse")
    n = grad.shape[0]
    if n_unique is not None:
        n_unique = _dev(n_unique, torch.int64, "n_unique")
    nb = lib().segsum_adam_workspace_bytes(n, u_max, table.dim)
    ws = _workspace("segsum_adam", nb, grad.device)
    _check(lib().emb_grad_segment_sum_adam(table.handle, _ptr(slots), _ptr(grad), _ptr(inverse), n,
                                           _ptr(n_unique), u_max, lr, b1, b2, eps, step, _ptr(ws), nb,
                                           _stream()))


# ----------------------------------------------------------------- helpers --
_hip = None


def _hip_lib():
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise ImportError("libamdhip64 not found")
        _hip.hipMemcpyAsync.argtypes = [_P, _P, _SZ, _I32, _P]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    return _hip


def copy_from_device_ptr(dst: torch.Tensor, src_ptr: int):
    """Device-to-device copy of dst.nbytes bytes from a raw device pointer into dst."""
    rc = _hip_lib().hipMemcpyAsync(dst.data_ptr(), src_ptr, dst.numel() * dst.element_size(), 3,
                                   _stream())
    if rc != 0:
        raise HTLError(HTL_ERR_DEVICE, f"hipMemcpyAsync failed ({rc})")
    return dst


def copy_to_device_ptr(dst_ptr: int, src: torch.Tensor):
    src = src.contiguous()
    rc = _hip_lib().hipMemcpyAsync(dst_ptr, src.data_ptr(), src.numel() * src.element_size(), 3,
                                   _stream())
    if rc != 0:
        raise HTLError(HTL_ERR_DEVICE, f"hipMemcpyAsync failed ({rc})")


def debug_build() -> bool:
    """Whether the loaded library is the debug build (device-side checks)."""
    return bool(lib().htl_debug_build())


def debug_flags() -> int:
    """The current device's invariant-violation bits (HTL_DEBUG_*; always 0
    in a release build), cleared by reading them; synchronises the device."""
    f = _U32(0)
    _check(lib().htl_debug_flags(ctypes.byref(f)))
    return int(f.value)


DEBUG_SLOT, DEBUG_DUP, DEBUG_WALK, DEBUG_FULL, DEBUG_DEDUP, DEBUG_LOG = 1, 2, 4, 8, 16, 32


def table_keys(table: Table) -> torch.Tensor:
    """A copy of the table's key array (int64[M])."""
    v = table.view()
    out = torch.empty(table.capacity, dtype=torch.int64, device=table.device)
    return copy_from_device_ptr(out, v.keys)


def table_tensor(table: Table, which: str) -> torch.Tensor:
    """A copy of 'rows' ([M, dim]), 'last_seen' ([M]), 'adam_m' or 'adam_v' ([M, dim]),
    'keys' ([M]) or, for a growable table, 'row_of_slot' ([M])."""
    v = table.view()
    M, d = table.capacity, table.dim
    if which == "keys":
        out = torch.empty(M, dtype=torch.int64, device=table.device)
        ptr = v.keys
    elif which == "row_of_slot":
        out = torch.empty(M, dtype=torch.int32, device=table.device)
        ptr = v.row_of_slot
    elif which == "rows":
        out = torch.empty((M, d), dtype=table.row_dtype, device=table.device)
        ptr = v.rows
    elif which == "last_seen":
        out = torch.empty(M, dtype=torch.int32, device=table.device)
        ptr = v.last_seen
    elif which in ("adam_m", "adam_v"):
        out = torch.empty((M, d), dtype=torch.float32, device=table.device)
        ptr = getattr(v, which)
    else:
        raise ValueError(which)
    if not ptr:
        raise ValueError(f"table keeps no {which}")
    return copy_from_device_ptr(out, ptr)
