"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function include/htl.h declares, size
its workspaces, and reject bad arguments with HTL_ERR_INVALID before it
touches the device.  No compute call is made here.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "htl.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def L():
    import hash_table_lookup_amd as h
    return h.lib()


# The C ABI proposed for the lookup path: every one of these calls must be
# declared and exported under its name.
BOUNDARY_CALLS = ("ht_create", "ht_destroy", "ht_find_or_insert", "ht_erase", "dedup_workspace_bytes",
                  "dedup_unique_inverse", "emb_gather_pool", "segsum_workspace_bytes", "emb_grad_segment_sum",
                  "emb_rowwise_adam", "ht_scan", "ht_rows", "htl_last_error")


def test_header_declares_the_boundary():
    names = _declared_functions()
    missing = [c for c in BOUNDARY_CALLS if c not in names]
    assert not missing, missing


def test_boundary_signatures():
    # argument lists of the boundary calls as the header declares them
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)

    def args(name):
        m = re.search(r"\b" + name + r"\s*\(([^;]*?)\)\s*;", src, flags=re.S)
        assert m, name
        return [" ".join(a.split()) for a in m.group(1).split(",")]

    assert args("ht_rows") == ["const htl_table* t", "const void** rows", "int64_t* row_bytes"]
    assert args("ht_scan") == ["const htl_table* t", "int64_t* keys", "uint32_t* last_seen", "int32_t* slots",
                               "int64_t* n_live_dev", "hipStream_t stream"]
    assert args("dedup_unique_inverse")[:5] == ["const int64_t* keys", "int64_t n", "int64_t* unique",
                                                "int32_t* inverse", "int64_t* n_unique_dev"]
    assert args("emb_gather_pool") == ["const htl_table* t", "const int32_t* slots", "const int32_t* inverse",
                                       "int64_t n", "const int32_t* offsets", "int64_t nbags",
                                       "htl_dtype out_dtype", "void* out", "hipStream_t stream"]
    assert args("segsum_workspace_bytes") == ["int64_t n", "int64_t u_max", "int dim"]


def test_rows_view_rejects_a_null_table(L):
    import ctypes as C
    p, rb = C.c_void_p(), C.c_int64(-1)
    assert L.ht_rows(None, C.byref(p), C.byref(rb)) == 1
    assert b"null table" in L.htl_last_error()


def test_every_declared_symbol_is_exported(L):
    import hash_table_lookup_amd as h
    names = _declared_functions()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(h.EXPORTED)


def test_workspace_sizes(L):
    a = L.dedup_workspace_bytes(1000)
    b = L.dedup_workspace_bytes(1 << 22)
    assert 0 < a < b and b % 256 == 0
    assert L.dedup_workspace_bytes(0) > 0
    s1 = L.segsum_workspace_bytes(1 << 20, 1 << 18, 128)
    s2 = L.segsum_workspace_bytes(1 << 20, 1 << 18, 64)
    assert s1 > s2 > 0
    # the fused backward needs no more than the segment-sum, except where rows
    # are not 16-byte vectors and the summed gradient goes through it
    assert L.segsum_adam_workspace_bytes(1 << 20, 1 << 18, 128) == s1
    assert L.segsum_adam_workspace_bytes(1 << 20, 1 << 18, 6) >= \
        L.segsum_workspace_bytes(1 << 20, 1 << 18, 6) + (1 << 18) * 6 * 4
    assert L.lru_workspace_bytes(None) == 0


def test_invalid_arguments_rejected_on_host(L):
    INVALID = 1
    h = ctypes.c_void_p()
    assert L.ht_create(None, 10, 16, 0, 0, 0, None) == INVALID
    assert L.ht_create(ctypes.byref(h), 0, 16, 0, 0, 0, None) == INVALID
    assert b"capacity_log2" in L.htl_last_error()
    assert L.ht_create(ctypes.byref(h), 32, 16, 0, 0, 0, None) == INVALID
    assert L.ht_create(ctypes.byref(h), 10, 0, 0, 0, 0, None) == INVALID
    assert L.ht_create(ctypes.byref(h), 10, 16, 7, 0, 0, None) == INVALID
    assert L.ht_create(ctypes.byref(h), 10, 16, 1, 0, 2, None) == INVALID   # Adam needs fp32
    assert L.ht_create(ctypes.byref(h), 10, 16, 0, 0, 16, None) == INVALID   # unknown flag
    assert L.ht_create(ctypes.byref(h), 10, 16, 0, 0, 8, None) == INVALID    # access log without last_seen
    assert b"access log" in L.htl_last_error()
    assert L.ht_create(ctypes.byref(h), 31, 16, 0, 0, 9, None) == INVALID    # access log above 2^30 slots
    assert L.ht_access_log_state(None, None, None) == INVALID
    assert L.ht_access_log_rebuild(None, None) == INVALID
    assert not h.value
    assert L.ht_find_or_insert(None, None, 4, None, 0, None, None, None) == INVALID
    assert L.ht_erase(None, None, 4, None, None) == INVALID
    assert L.ht_scan(None, None, None, None, None, None) == INVALID
    assert L.dedup_unique_inverse(None, -1, None, None, None, None, 0, None) == INVALID
    assert L.dedup_unique_inverse(None, 1 << 31, None, None, None, None, 0, None) == INVALID
    assert L.emb_gather_pool(None, None, None, 1, None, 0, 0, None, None) == INVALID
    assert L.emb_grad_segment_sum(None, None, 10, None, 11, 4, None, None, 0, None) == INVALID
    assert L.emb_grad_segment_sum(None, None, (1 << 31) - 1024, None, 1, 4, None, None, 0, None) == INVALID
    assert L.emb_grad_segment_sum(None, None, 10, None, 5, 0, None, None, 0, None) == INVALID
    assert L.emb_rowwise_adam(None, None, None, 1, None, 1e-3, 0.9, 0.999, 1e-8, 1, None) == INVALID
    assert L.emb_grad_segment_sum_adam(None, None, None, None, 10, None, 5, 1e-3, 0.9, 0.999, 1e-8, 1,
                                       None, 0, None) == INVALID
    assert L.ht_lru_select(None, 1, 20, None, 0, None, None, 0, None) == INVALID
    assert L.ht_resize(None, 10, None) == INVALID
    assert L.ht_export(None, 0, 1, None, None, None, None, None, None, None) == INVALID
    assert L.ht_import(None, None, 1, None, None, None, None, None, None) == INVALID
    assert L.ht_view(None, None) == INVALID
    assert L.emb_lookup_slots(None, None, 4, 0, None, None, None, None, None, None, None, 0, None) == INVALID
    assert L.emb_lookup(None, None, 4, 0, None, None, None, None, None, None, 0, 0, None, None, 0, None) == INVALID
    assert L.emb_lookup_workspace_bytes(1 << 20) >= L.dedup_workspace_bytes(1 << 20) + 4 * (1 << 20)
    assert L.ht_destroy(None) == 0
    fake = ctypes.c_void_p(0x1000)
    assert L.htl_copy_probe(fake, fake, 24, None) == INVALID            # not a multiple of 16
    assert L.htl_copy_probe(fake, ctypes.c_void_p(0x1008), 32, None) == INVALID   # misaligned
    assert L.htl_copy_probe(None, None, 0, None) == 0                   # nothing to copy


def test_misaligned_workspace_rejected(L):
    INVALID = 1
    # host-visible checks only: a bogus but non-null pointer is never dereferenced
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1001)
    n_dev = ctypes.c_void_p(0x2000)
    assert L.dedup_unique_inverse(fake, 10, fake, fake, n_dev, odd, 1 << 20, None) == INVALID
    assert L.dedup_unique_inverse(fake, 10, fake, fake, n_dev, fake, 16, None) == INVALID
    assert b"workspace" in L.htl_last_error()


def test_noalloc_dedup_limit_checked_on_the_host(L):
    # beyond 2^20 keys the allocation-free dedup refuses before touching a device
    assert L.dedup_noalloc_max_keys() == 1 << 20
    fake = ctypes.c_void_p(0x1000)
    assert L.dedup_unique_inverse_noalloc(fake, (1 << 20) + 1, fake, fake, fake, None) == 1
    assert b"2^20" in L.htl_last_error()
    assert L.dedup_unique_inverse_noalloc(fake, -1, fake, fake, fake, None) == 1


def test_adaptive_dedup_host_checks(L):
    # no plan: refused before anything is enqueued; the choice without a plan
    # is the batch-size default
    fake = ctypes.c_void_p(0x1000)
    assert L.dedup_unique_inverse_adaptive(None, fake, 10, fake, fake, fake, fake, 1 << 20, None) == 1
    assert L.dedup_plan_stats(None, None) == 1
    assert L.dedup_plan_destroy(None) == 0
    assert L.dedup_plan_choose(None, 100) == 0
    assert L.dedup_plan_choose(None, 1 << 20) == 1
    assert L.dedup_plan_choose(None, (1 << 23) + 1) == 3


def test_debug_build_reports_itself(L):
    # the release library is no debug build; the debug variant (if built)
    # says it is -- a host-only call in both
    assert L.htl_debug_build() == 0
    dbg = os.path.join(ROOT, "hash_table_lookup_amd", "libhtl_debug.so")
    if not os.path.exists(dbg):
        pytest.skip("libhtl_debug.so not built")
    D = ctypes.CDLL(dbg)
    assert D.htl_debug_build() == 1
    assert D.htl_debug_flags(None) == 1                   # null output: INVALID, before any device call
