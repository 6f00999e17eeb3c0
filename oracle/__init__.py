"""ctypes wrapper of the CPU oracle (oracle.cpp) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package.  The HIP library and its Python
binding never do, and share no code with it.

The oracle is plain single-threaded C++ built with ``g++ -O2
-ffp-contract=off`` into ``oracle/liboracle.so`` by :func:`build`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
# The same source built with AddressSanitizer and UndefinedBehaviorSanitizer;
# HTL_ORACLE_LIB loads it (with gcc's ASan runtime preloaded) in place of
# liboracle.so.
SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")

FOUND, INSERTED, FULL, RESERVED = 0, 1, 2, 3
NOT_FOUND, ERASED = 0, 1
F32, BF16 = 0, 1
EMPTY_KEY, TOMBSTONE_KEY = -1, -2


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile liboracle.so with g++ (single-threaded, no FP contraction);
    sanitize: liboracle_san.so under ASan + UBSan."""
    out = SAN_LIB_PATH if sanitize else LIB_PATH
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp"
        cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp]
        if sanitize:
            cmd[3:3] = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("HTL_ORACLE_LIB")
        if not path:
            if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
                build()
            path = LIB_PATH
        L = ctypes.CDLL(path)
        sig = {
            "orc_mix64": (_U64, [_U64]),
            "orc_splitmix64": (None, [_U64, _I64, _P]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_init_row": (None, [_I64, _U64, _I32, _I32, _P]),
            "orc_probe_coverage": (_I64, [_U64, _U64, _U64]),
            "orc_bucket_probe_coverage": (_I64, [_U64, _U64, _U64, _U64]),
            "orc_dedup": (_I64, [_P, _I64, _P, _P]),
            "orc_table_create": (_P, [_I64, _I32, _I32, _U64, _I32]),
            "orc_table_destroy": (None, [_P]),
            "orc_table_size": (_I64, [_P]),
            "orc_table_resize": (_I32, [_P, _I64]),
            "orc_find_or_insert": (None, [_P, _P, _I64, _U32, _P]),
            "orc_erase": (None, [_P, _P, _I64, _P]),
            "orc_lookup": (_I32, [_P, _I64, _P, _P, _P, _P]),
            "orc_gather": (None, [_P, _P, _I64, _P]),
            "orc_gather_pool": (None, [_P, _P, _P, _I64, _I32, _P]),
            "orc_segment_sum": (None, [_P, _P, _I64, _I64, _I32, _P, _P]),
            "orc_adam": (None, [_P, _P, _P, _I64, ctypes.c_float, ctypes.c_float,
                                ctypes.c_float, ctypes.c_float, _I64]),
            "orc_adam_arrays": (None, [_P, _P, _P, _P, _I64, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, _I64]),
            "orc_adam_arrays_f32": (None, [_P, _P, _P, _P, _I64, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_float, _I64]),
            "orc_live": (_I64, [_P, _P, _P]),
            "orc_lru_victims": (_I64, [_P, _I64, _I64, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- primitives
def mix64(x: int) -> int:
    return int(lib().orc_mix64(x & 0xFFFFFFFFFFFFFFFF))


def splitmix64(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().orc_splitmix64(seed & 0xFFFFFFFFFFFFFFFF, n, _ptr(out))
    return out


def f32_to_bf16_bits(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(x)))


def init_row(key: int, dim: int, dtype: int = F32, seed: int = 0) -> np.ndarray:
    """Closed-form initial row: float32[dim], or uint16 bf16 bits[dim]."""
    out = np.empty(dim, dtype=np.float32 if dtype == F32 else np.uint16)
    lib().orc_init_row(int(key), seed & 0xFFFFFFFFFFFFFFFF, dim, dtype, _ptr(out))
    return out


def init_rows(keys, dim: int, dtype: int = F32, seed: int = 0) -> np.ndarray:
    keys = np.asarray(keys, dtype=np.int64)
    out = np.empty((keys.size, dim), dtype=np.float32 if dtype == F32 else np.uint16)
    for i, k in enumerate(keys):
        lib().orc_init_row(int(k), seed & 0xFFFFFFFFFFFFFFFF, dim, dtype, _ptr(out[i]))
    return out


# ------------------------------------------------------------------ theorem 1
def probe_coverage(M: int, h0: int, S: int) -> int:
    return int(lib().orc_probe_coverage(M, h0, S))


def bucket_probe_coverage(M: int, W: int, b0: int, S: int) -> int:
    return int(lib().orc_bucket_probe_coverage(M, W, b0, S))


# ---------------------------------------------------------------------- dedup
def dedup(keys):
    """(unique sorted int64 [U], inverse int32 [N])."""
    keys = _c(keys, np.int64)
    uniq = np.empty(keys.size, dtype=np.int64)
    inv = np.empty(keys.size, dtype=np.int32)
    u = lib().orc_dedup(_ptr(keys), keys.size, _ptr(uniq), _ptr(inv))
    return uniq[:u].copy(), inv


def segment_sum(grad, inverse, n_unique: int, want_abs: bool = True):
    """(fp64 sums [U, D], fp64 sums of |g| [U, D] or None)."""
    grad = _c(grad, np.float32)
    inverse = _c(inverse, np.int32)
    n, d = grad.shape
    s = np.empty((n_unique, d), dtype=np.float64)
    a = np.empty((n_unique, d), dtype=np.float64) if want_abs else None
    lib().orc_segment_sum(_ptr(grad), _ptr(inverse), n, n_unique, d, _ptr(s),
                          _ptr(a) if a is not None else None)
    return s, a


def adam_arrays(theta, m, v, g, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, step=1):
    """One Adam step on copies of fp32 arrays; returns (theta, m, v)."""
    th = np.array(theta, dtype=np.float32, copy=True, order="C")
    mm = np.array(m, dtype=np.float32, copy=True, order="C")
    vv = np.array(v, dtype=np.float32, copy=True, order="C")
    gg = _c(g, np.float32)
    assert th.shape == mm.shape == vv.shape == gg.shape
    lib().orc_adam_arrays(_ptr(th), _ptr(mm), _ptr(vv), _ptr(gg), th.size, lr, b1, b2, eps, step)
    return th, mm, vv


def adam_arrays_f32(theta, m, v, g, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, step=1):
    """One Adam step evaluated in fp32, each operation rounded as written;
    returns (theta, m, v)."""
    th = np.array(theta, dtype=np.float32, copy=True, order="C")
    mm = np.array(m, dtype=np.float32, copy=True, order="C")
    vv = np.array(v, dtype=np.float32, copy=True, order="C")
    gg = _c(g, np.float32)
    assert th.shape == mm.shape == vv.shape == gg.shape
    lib().orc_adam_arrays_f32(_ptr(th), _ptr(mm), _ptr(vv), _ptr(gg), th.size, lr, b1, b2, eps, step)
    return th, mm, vv


# ---------------------------------------------------------------------- table
class Table:
    """The oracle's dynamic embedding table (a std::unordered_map)."""

    def __init__(self, capacity: int, dim: int, dtype: int = F32, seed: int = 0,
                 adam: bool = False):
        self.capacity, self.dim, self.dtype, self.seed = capacity, dim, dtype, seed
        self._h = lib().orc_table_create(capacity, dim, dtype, seed & 0xFFFFFFFFFFFFFFFF,
                                         1 if adam else 0)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_table_destroy(h)
            self._h = None

    @property
    def row_dtype(self):
        return np.float32 if self.dtype == F32 else np.uint16

    def __len__(self):
        return int(lib().orc_table_size(self._h))

    def resize(self, capacity: int):
        """Raise the capacity (live keys keep their rows and metadata)."""
        if not lib().orc_table_resize(self._h, capacity):
            raise ValueError("capacity below the live count")
        self.capacity = capacity

    def find_or_insert(self, keys, step: int = 0) -> np.ndarray:
        keys = _c(keys, np.int64)
        st = np.empty(keys.size, dtype=np.uint8)
        lib().orc_find_or_insert(self._h, _ptr(keys), keys.size, step, _ptr(st))
        return st

    def erase(self, keys) -> np.ndarray:
        keys = _c(keys, np.int64)
        st = np.empty(keys.size, dtype=np.uint8)
        lib().orc_erase(self._h, _ptr(keys), keys.size, _ptr(st))
        return st

    def lookup(self, key: int):
        """(row, last_seen, m, v) or None if the key is not live."""
        row = np.empty(self.dim, dtype=self.row_dtype)
        ls = np.empty(1, dtype=np.uint32)
        m = np.empty(self.dim, dtype=np.float32)
        v = np.empty(self.dim, dtype=np.float32)
        ok = lib().orc_lookup(self._h, int(key), _ptr(row), _ptr(ls), _ptr(m), _ptr(v))
        return (row, int(ls[0]), m, v) if ok else None

    def gather(self, keys) -> np.ndarray:
        keys = _c(keys, np.int64)
        out = np.empty((keys.size, self.dim), dtype=self.row_dtype)
        lib().orc_gather(self._h, _ptr(keys), keys.size, _ptr(out))
        return out

    def gather_pool(self, keys, offsets, out_dtype: int = F32) -> np.ndarray:
        keys = _c(keys, np.int64)
        offsets = _c(offsets, np.int32)
        nb = offsets.size - 1
        out = np.empty((nb, self.dim), dtype=np.float32 if out_dtype == F32 else np.uint16)
        lib().orc_gather_pool(self._h, _ptr(keys), _ptr(offsets), nb, out_dtype, _ptr(out))
        return out

    def adam(self, keys, g, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, step=1):
        keys = _c(keys, np.int64)
        g = _c(g, np.float32)
        lib().orc_adam(self._h, _ptr(keys), _ptr(g), keys.size, lr, b1, b2, eps, step)

    def live(self):
        """(keys ascending int64, last_seen uint32)."""
        n = len(self)
        k = np.empty(n, dtype=np.int64)
        ls = np.empty(n, dtype=np.uint32)
        lib().orc_live(self._h, _ptr(k), _ptr(ls))
        return k, ls

    def lru_victims(self, num: int, den: int) -> np.ndarray:
        out = np.empty(max(len(self), 1), dtype=np.int64)
        k = lib().orc_lru_victims(self._h, num, den, _ptr(out))
        return out[:k].copy()


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)
