"""The debug build (libhtl_debug.so, -DHTL_DEBUG): after each find-or-insert,
dedup and logged erase it checks the table's invariants on the device and
records violations as flag bits (htl_debug_flags).

Run in a child process that loads the debug library in place of libhtl.so:
an online stream on a logged table, a growable table with a resize and
dedups of several sizes must leave every flag clear; then a duplicate key
written into the key array from the host (as a caller writing through
ht_view could) must be reported by the next find-or-insert of that key.
No kernel is made to fault: the planted state is an ordinary key value in
an empty slot of the key's own bucket.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "hash_table_lookup_amd", "libhtl_debug.so")

pytestmark = pytest.mark.gpu

CHILD = r"""
import numpy as np, torch
import hash_table_lookup_amd as htl, workloads
assert htl.debug_build(), "not the debug library"
torch.cuda.set_device(0)

# an online stream on a logged table: forward, eviction, erase
spec = workloads.DynamicOnlineSpec(window=1 << 13, n=1 << 12, capacity_log2=16, dim=8)
t = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, access_log=True)
for s in range(6):
    keys = torch.from_numpy(workloads.dynamic_online_step(spec, s)).cuda()
    htl.lookup(t, keys, step=s, fused=(s % 2 == 0))
    v, nv = t.lru_select(spec.evict_num, spec.evict_den)
    t.erase(v[:int(nv.item())])
print("online flags", htl.debug_flags(), flush=True)

# a growable table, resized, and a small full table
g = htl.Table(12, 4, "f32", growable=True)
rng = np.random.default_rng(1)
for s in range(3):
    g.find_or_insert(torch.from_numpy(np.unique(rng.integers(0, 1 << 40, 2000))).cuda())
    if s == 1:
        g.resize(14)
f = htl.Table(5, 4, "f32")
f.find_or_insert(torch.arange(100, dtype=torch.int64, device="cuda"))      # 32 slots: FULL for the rest
for n in (1000, 100_003, 1 << 20):
    htl.dedup_unique_inverse(torch.from_numpy(rng.integers(0, n // 3 + 1, n)).cuda())
clean = htl.debug_flags()
print("clean flags", clean, flush=True)
assert clean == 0, clean

# a second copy of a live key, in a free slot of its own bucket
d = htl.Table(10, 4, "f32")
ks = np.arange(1, 200, dtype=np.int64) * 1_000_003
d.find_or_insert(torch.from_numpy(ks).cuda())
assert htl.debug_flags() == 0
tk = htl.table_keys(d).cpu().numpy()
planted = False
for s in np.flatnonzero(tk >= 0):
    b0 = s - s % 16
    free = [j for j in range(b0, b0 + 16) if tk[j] == -1]
    if free:
        k = int(tk[s])
        htl.copy_to_device_ptr(d.view().keys + 8 * free[0], torch.tensor([k], dtype=torch.int64, device="cuda"))
        torch.cuda.synchronize()
        d.find_or_insert(torch.tensor([k], dtype=torch.int64, device="cuda"))
        planted = True
        break
assert planted
got = htl.debug_flags()
print("planted flags", got, flush=True)
assert got & htl.DEBUG_DUP, got
print("OK", flush=True)
"""


@pytest.mark.skipif(not os.path.exists(DEBUG_LIB), reason="libhtl_debug.so not built (python -m hash_table_lookup_amd.build --debug)")
def test_debug_build_checks():
    env = dict(os.environ, HTL_LIB=DEBUG_LIB, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, cwd=ROOT, capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and "OK" in r.stdout
