"""Benchmark of the sparse-embedding lookup hot path on one MI355X.

A step is one pass of the forward hot path over one batch: two-stage dedup
-> find-or-insert of the unique keys into the dynamic table (misses inserted)
-> per-ID row gather, as dedup_unique_inverse -> ht_find_or_insert ->
emb_gather_pool.  The default workload is the large-table lookup: 2^22 IDs
drawn Zipf(1.05) over a 2^40 key universe against a 2^24-slot fp32 table of
dim 64 pre-filled (untimed) with the 2^23 most popular keys.

Timing: each step is bracketed by HIP events on the stream the library
launches on; between steps the table's key array is restored to its
pre-filled state by a device-to-device copy that lies outside the events, so
every step sees the same table.  The K timed steps as a whole are also
bracketed by torch.cuda.synchronize() and reported as wall time (restores
included).  value = IDs per second over the hot path (Mkeys/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, AMD's published peak
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "hash_table_lookup_amd", "csrc")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gather_single_large_table_traffic.txt")
TRAFFIC_SOURCES = [os.path.join(CSRC, f) for f in ("gather.hip", "htl_common.h")]


def _measured_traffic():
    """Counter-measured HBM bytes per gather launch, or None if the gather's
    source changed since the counters were taken (or no record exists)."""
    import hashlib
    record, sources = TRAFFIC_RECORD, TRAFFIC_SOURCES
    try:
        rec = {}
        for line in open(record):
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in sources:
            h.update(open(f, "rb").read())
        if h.hexdigest() != rec.get("source_sha256"):
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="single_large_table",
                    choices=["single_large_table", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1 << 22,
                    help="IDs of the batch the CPU oracle processes (timed)")
    return ap.parse_args()


def _algorithmic_bytes(n, U, hits, misses, dim, esz):
    """Minimum HBM bytes of the whole path and of its gather kernel.

    Whole path: per ID 8 (key read) + 4 (inverse write) + 4 (inverse read) +
    row (output); per unique key 8 (unique write) + 8 (unique read) + 4 + 4
    (slot write/read) + 1 (status) + 8 (table key probe); per hit one row
    read; per miss one key claim (8) and one initial-row write.
    Gather kernel (k_gather): per ID 4 (inverse) + row (output); per unique
    4 (slot) + row (read).
    """
    row = dim * esz
    path = n * (8 + 4 + 4 + row) + U * (8 + 8 + 4 + 4 + 1 + 8) + hits * row + misses * (8 + row)
    gather = n * (4 + row) + U * (4 + row)
    return path, gather


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the sharded design is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import hash_table_lookup_amd as htl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.workload == "single_large_table":
        w = workloads.single_large_table()
    else:
        w = workloads.tiny()
    n = w.keys.size
    keys = torch.from_numpy(w.keys).to(dev)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    if w.prefill is not None:
        _, st = table.find_or_insert(torch.from_numpy(w.prefill).to(dev))
        assert bool((st == htl.INSERTED).all())
    saved_keys = htl.table_keys(table).clone()
    view = table.view()
    stream = torch.cuda.current_stream()

    def restore():
        htl._binding.copy_to_device_ptr(view.keys, saved_keys)

    # outputs preallocated once: the timed region allocates nothing
    out = torch.empty((n, w.dim), dtype=table.row_dtype, device=dev)

    def step(e_gather=None):
        """One pass of the hot path; records e_gather just before the gather kernel."""
        uniq, inv, nu = htl.dedup_unique_inverse(keys)
        slots, status = table.find_or_insert(uniq, n_dev=nu)
        if e_gather is not None:
            e_gather.record(stream)
        htl.gather(table, slots, inv, out=out)
        return uniq, inv, nu, slots, status

    for _ in range(args.warmup):
        step()
        restore()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e_start, e_gather, e_end = ev[i]
        e_start.record(stream)
        uniq, inv, nu, slots, status = step(e_gather)
        e_end.record(stream)
        restore()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    step_ms = np.array([a.elapsed_time(c) for a, b, c in ev])
    gather_ms = np.array([b.elapsed_time(c) for a, b, c in ev])
    U = int(nu.item())
    st = status[:U]
    hits = int((st == htl.FOUND).sum().item())
    misses = int((st == htl.INSERTED).sum().item())
    esz = 4 if w.dtype == "f32" else 2
    path_bytes, gather_bytes = _algorithmic_bytes(n, U, hits, misses, w.dim, esz)
    mean_ms = float(step_ms.mean())
    mkeys = n / (mean_ms * 1e-3) / 1e6
    g_ms = float(gather_ms.mean())
    g_gbs = gather_bytes / (g_ms * 1e-3) / 1e9

    result = {
        "metric": "dedup+lookup+gather Mkeys/s and achieved HBM GB/s vs peak on 1 MI355X",
        "value": round(mkeys, 2),
        "unit": "Mkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64 keys, " + ("fp32" if w.dtype == "f32" else "bf16") + " rows",
        "data": "synthetic: seeded Zipf ID stream (numpy PCG64), closed-form table rows",
        "config": {
            "workload": w.name,
            "ids_per_step": n,
            "zipf_a": w.meta.get("zipf_a"),
            "key_universe_log2": w.meta.get("universe_log2"),
            "table_slots_log2": w.capacity_log2,
            "prefilled_keys": 0 if w.prefill is None else int(w.prefill.size),
            "dim": w.dim,
            "row_dtype": w.dtype,
            "parallelism": "single GPU",
        },
        "path": {
            "unique": U, "hits": hits, "misses": misses,
            "hit_rate_per_id": None,
            "algorithmic_bytes": path_bytes,
            "achieved_gbs": round(path_bytes / (mean_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(path_bytes / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_median": round(float(np.median(step_ms)), 4),
            "wall_ms_per_step_incl_restore": round(wall / args.steps * 1e3, 4),
            "implementation": "dedup_unique_inverse + ht_find_or_insert + emb_gather_pool",
            "timing": "HIP events around dedup+find_or_insert+gather per step on the launch stream; "
                      "table keys restored by a D2D copy between steps, outside the events",
        },
        "roofline": {
            "kernel": "k_gather (emb_gather_pool: per-ID rows)",
            "bound": "hbm",
            "achieved": round(g_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(g_gbs / HBM_PEAK_GBS, 4),
            "traffic": _measured_traffic() if w.name == "single_large_table" else None,
            "algorithmic_bytes_per_launch": gather_bytes,
            "avg_launch_ms": round(g_ms, 4),
        },
    }
    # hit rate per ID: fraction of IDs whose key was FOUND
    found_map = torch.zeros(U, dtype=torch.bool, device=dev)
    found_map[:] = st == htl.FOUND
    result["path"]["hit_rate_per_id"] = round(float(found_map[inv.long()].float().mean().item()), 4)

    result["copy_reference"] = _copy_reference(torch, htl, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(w, args.cpu_sample)
    print(json.dumps(result), flush=True)


def _copy_reference(torch, htl, dev, nbytes=1 << 30, reps=5):
    """Achievable streaming bandwidth: a 1 GiB device-to-device copy (read + write)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        htl._binding.copy_to_device_ptr(dst.data_ptr(), src)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    gbs = 2 * nbytes / (best * 1e-3) / 1e9
    return {"kind": "hipMemcpyAsync device-to-device, 1 GiB", "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def _cpu_baseline(w, sample):
    """The oracle timed on the host (single thread) on the first `sample` IDs."""
    import oracle
    m = min(sample, w.keys.size)
    keys = np.ascontiguousarray(w.keys[:m])
    tab = oracle.Table(1 << w.capacity_log2, w.dim, oracle.F32 if w.dtype == "f32" else oracle.BF16)
    if w.prefill is not None:
        tab.find_or_insert(w.prefill)
    t0 = time.perf_counter()
    uniq, inv = oracle.dedup(keys)
    tab.find_or_insert(uniq)
    tab.gather(keys)
    dt = time.perf_counter() - t0
    return {"value": round(m / dt / 1e6, 3), "unit": "Mkeys/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m} IDs of the same batch, dedup+find_or_insert+gather, table pre-filled "
                      f"untimed; {dt:.2f} s", "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
