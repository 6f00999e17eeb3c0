"""The allocation-free dedup entry point (dedup_unique_inverse_noalloc),
called through the C ABI and compared with dedup_unique_inverse on the same
keys: the same unique count and set, an inverse that maps every ID back to
its key, and the canonical (sorted-rank) inverse equal to the oracle's.

Two calls run back to back, the second on a smaller batch, so that the
second call works in a scratch array that still holds the first call's
state; both must match the workspace entry point exactly in what the dedup
defines.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from conftest import to_np

pytestmark = pytest.mark.gpu


def _noalloc(htl, keys):
    n = keys.numel()
    unique = torch.empty(max(n, 1), dtype=torch.int64, device=keys.device)
    inverse = torch.empty(max(n, 1), dtype=torch.int32, device=keys.device)
    nu = torch.full((1,), -7, dtype=torch.int64, device=keys.device)
    L = htl.lib()
    st = L.dedup_unique_inverse_noalloc(ctypes.c_void_p(keys.data_ptr()), n, ctypes.c_void_p(unique.data_ptr()),
                                        ctypes.c_void_p(inverse.data_ptr()), ctypes.c_void_p(nu.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.htl_last_error()
    return unique, inverse[:n], nu


def _same_dedup(htl, orc, keys_np):
    keys = torch.from_numpy(keys_np).cuda()
    ua, ia, na = _noalloc(htl, keys)
    ub, ib, nb = htl.dedup_unique_inverse(keys)
    torch.cuda.synchronize()
    U = int(na.item())
    assert U == int(nb.item())
    ref_u, ref_inv = orc.dedup(keys_np)
    assert U == ref_u.size
    a, b = to_np(ua)[:U], to_np(ub)[:U]
    assert np.array_equal(np.sort(a), ref_u) and np.array_equal(np.sort(b), ref_u)
    if keys_np.size:
        ia_np, ib_np = to_np(ia), to_np(ib)
        assert np.array_equal(a[ia_np], keys_np) and np.array_equal(b[ib_np], keys_np)
        assert np.array_equal(np.searchsorted(ref_u, a[ia_np]).astype(np.int32), ref_inv)


@pytest.mark.parametrize("sizes", [(300_000, 70_001), (1 << 20, 2049), (2048, 0), (100_003, 1)])
def test_noalloc_dedup_two_calls_second_smaller(htl, orc, sizes):
    for i, n in enumerate(sizes):
        w = workloads.tiny(seed=11 + i, n=max(n, 1))
        _same_dedup(htl, orc, w.keys[:n])


def test_noalloc_dedup_on_the_device_set_path(htl, orc, monkeypatch):
    # the other form of the second stage uses the same scratch
    monkeypatch.setenv("HTL_DEDUP_PATH", "set")
    for i, n in enumerate((500_000, 9_999)):
        w = workloads.tiny(seed=21 + i, n=n)
        _same_dedup(htl, orc, w.keys)


def test_noalloc_dedup_rejects_more_than_its_limit(htl):
    L = htl.lib()
    m = L.dedup_noalloc_max_keys()
    assert m == 1 << 20
    keys = torch.zeros(m + 1, dtype=torch.int64, device="cuda")
    out = torch.empty(m + 1, dtype=torch.int64, device="cuda")
    inv = torch.empty(m + 1, dtype=torch.int32, device="cuda")
    nu = torch.empty(1, dtype=torch.int64, device="cuda")
    st = L.dedup_unique_inverse_noalloc(ctypes.c_void_p(keys.data_ptr()), m + 1, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(inv.data_ptr()), ctypes.c_void_p(nu.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 1 and b"2^20" in L.htl_last_error()
