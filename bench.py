"""Benchmark of the sparse-embedding lookup hot path on one MI355X.

Default workload (the one the headline metric is quoted on): the large-table
lookup -- 2^22 IDs drawn Zipf(1.05) over a 2^40 key universe against a
2^24-slot fp32 table of dim 64 pre-filled (untimed) with the 2^23 most popular
keys.  A step is one pass of the forward hot path over the batch:
dedup_unique_inverse -> ht_find_or_insert (misses inserted) ->
emb_gather_pool.

Other workloads (--workload), each its own hot-path rows:
  tiny            the same forward path, 65,536 IDs, 2^18-slot table
  merged_tables   26 tables merged into one 2^26-slot bf16 table (dim 128),
                  65,536 samples x 26 bags of Poisson(20) IDs: dedup ->
                  find-or-insert -> gather + sum-pool (bf16 out)
  backward        2^23 IDs Zipf(1.2), fp32 gradients [N, 128]: segment-sum
                  by the forward's inverse with row-wise Adam applied to each
                  finished row (one call; forward untimed); the two-call form
                  (segment-sum, then Adam) is timed beside it
  dynamic_online  2^27-slot bf16 table (dim 64), steps of 2^22 IDs over a
                  drifting window: dedup -> find-or-insert -> gather, then
                  LRU selection of 5% of the live keys and their erase;
                  with --growable the table keeps rows apart from its key
                  index and one capacity doubling (2^27 -> 2^28) is timed

Timing: HIP events on the stream the library launches on bracket each step
(and the dominant kernel inside it); table state that a step changes is
restored between steps outside the events (forward workloads), so every step
sees the same table.  The K timed steps are bracketed by
torch.cuda.synchronize() and reported as wall time too.

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
# Counter-measured bytes of each workload's roofline kernel (FETCH_SIZE and
# WRITE_SIZE: what the L2s exchange with the data fabric, Infinity Cache hits
# included, so an upper bound on HBM bytes), per record under profiles/,
# with the sources that decide them: the kernel's own, the
# dedup's (the order of unique ids it produces decides how the kernel's slot
# and row reads fall on cache lines), and for the row reads the probe header
# (how find-or-insert stores the new rows decides whether the gather finds
# them in L2).
_DEDUP_SRC = ("dedup.hip", "tile_dedup.h")
TRAFFIC_RECORDS = {
    "single_large_table": ("gather_single_large_table_traffic.txt", ("gather.hip",) + _DEDUP_SRC + ("probe.h",)),
    "merged_tables": ("pool_merged_tables_traffic.txt", ("pool.hip",) + _DEDUP_SRC + ("probe.h",)),
    "backward": ("backward_fused_traffic.txt", ("backward.hip", "scan.hip") + _DEDUP_SRC),
    "dynamic_online": ("gather_dynamic_online_traffic.txt", ("gather.hip",) + _DEDUP_SRC + ("probe.h",)),
}
METRIC = "dedup+lookup+gather Mkeys/s and achieved HBM GB/s vs peak on 1 MI355X"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="single_large_table",
                    choices=["single_large_table", "tiny", "merged_tables", "backward", "dynamic_online"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pcie", action="store_true",
                    help="skip the host-to-device overlap measurement of the large-table workload")
    ap.add_argument("--checkpoint", action="store_true",
                    help="dynamic_online: time a full export / host copy / import of the table")
    ap.add_argument("--growable", action="store_true",
                    help="dynamic_online: use a growable table and time one capacity doubling")
    ap.add_argument("--no-access-log", action="store_true",
                    help="dynamic_online: a table without the access log (eviction scans last_seen)")
    ap.add_argument("--cpu-sample", type=int, default=1 << 22,
                    help="IDs of the batch the CPU oracle processes (timed)")
    return ap.parse_args()


def _measured_traffic(workload):
    """Counter-measured L2-to-fabric bytes per launch of the workload's roofline
    kernel, or None if its sources or the dedup's changed since the counters
    were taken (or no record exists)."""
    import hashlib
    try:
        name, sources = TRAFFIC_RECORDS[workload]
        rec = {}
        for line in open(os.path.join(ROOT, "profiles", name)):
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in sources:
            h.update(open(os.path.join(CSRC, f), "rb").read())
        if h.hexdigest() != rec.get("source_sha256"):
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Timer:
    """Per-step HIP events (start, mark, end) on one stream."""

    def __init__(self, torch, steps):
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        self.ev = [(E(), E(), E()) for _ in range(steps)]

    def step_ms(self):
        return np.array([a.elapsed_time(c) for a, b, c in self.ev])

    def kernel_ms(self):
        return np.array([b.elapsed_time(c) for a, b, c in self.ev])


def _roofline(kernel, alg_bytes, ms, traffic=None):
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": int(alg_bytes), "avg_launch_ms": round(ms, 4)}


def _result(args, value, ms, config, dtype, path, roofline, unit="Mkeys/s"):
    return {"metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype,
            "data": "synthetic: seeded Zipf ID streams (numpy PCG64), closed-form table rows",
            "config": config, "path": path, "roofline": roofline}


def _lookup_bufs(torch, n, dev):
    """Output buffers of emb_lookup_slots, allocated once outside the timed steps."""
    return {"unique": torch.empty(n, dtype=torch.int64, device=dev),
            "inverse": torch.empty(n, dtype=torch.int32, device=dev),
            "n_unique": torch.empty(1, dtype=torch.int64, device=dev),
            "slots": torch.empty(n, dtype=torch.int32, device=dev),
            "status": torch.empty(n, dtype=torch.uint8, device=dev),
            "id_slots": torch.empty(n, dtype=torch.int32, device=dev)}


def _lookup_bytes(n, U, hits, misses, row):
    """Minimum HBM bytes of the forward path and of its gather kernel.

    Whole path: per ID 8 (key read) + 4 (inverse write) + 4 (inverse read) +
    row (output); per unique key 8 (unique write) + 8 (unique read) + 4 + 4
    (slot write/read) + 1 (status) + 8 (table key probe); per hit one row
    read; per miss one key claim (8) and one initial-row write.
    Gather kernel (k_gather over the per-ID slots): per ID 4 (its slot) + row
    (output); per unique key one row read.
    """
    path = n * (8 + 4 + 4 + row) + U * (8 + 8 + 4 + 4 + 1 + 8) + hits * row + misses * (8 + row)
    gather = n * (4 + row) + U * row
    return path, gather


def _statuses(htl, status, U):
    st = status[:U]
    return int((st == htl.FOUND).sum().item()), int((st == htl.INSERTED).sum().item())


def _timed(torch, args, step, restore=None):
    """Warm-up, then K steps with events; step(mark_event) runs one step."""
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step(None)
        if restore:
            restore()
    T = Timer(torch, args.steps)
    last = None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b, c in T.ev:
        a.record(stream)
        last = step(b)
        c.record(stream)
        if restore:
            restore()
    torch.cuda.synchronize()
    return T, time.perf_counter() - t0, last


# ------------------------------------------------------------------ forward
def run_lookup(args, torch, htl, workloads, dev):
    w = workloads.single_large_table() if args.workload == "single_large_table" else workloads.tiny()
    n = w.keys.size
    keys = torch.from_numpy(w.keys).to(dev)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    if w.prefill is not None:
        _, st = table.find_or_insert(torch.from_numpy(w.prefill).to(dev))
        assert bool((st == htl.INSERTED).all())
    saved_keys = htl.table_keys(table).clone()
    view = table.view()
    stream = torch.cuda.current_stream()
    # the outputs of the timed step are allocated once, here (the three-call
    # reference takes its unique, inverse, slots and status from torch's
    # caching allocator every step: no device allocation once it holds them)
    out = torch.empty((n, w.dim), dtype=table.row_dtype, device=dev)
    bufs = _lookup_bufs(torch, n, dev)

    def restore():
        htl._binding.copy_to_device_ptr(view.keys, saved_keys)

    def step(mark):
        # emb_lookup_slots (dedup, find-or-insert, each ID's slot), then the
        # gather over the per-ID slots -- the two halves of emb_lookup
        uniq, inv, nu, slots, status, ids = htl.lookup_slots(table, keys, bufs=bufs)
        if mark is not None:
            mark.record(stream)
        htl.gather(table, ids, None, out=out)
        return uniq, inv, nu, slots, status

    def three_calls(mark):
        uniq, inv, nu = htl.dedup_unique_inverse(keys)
        slots, status = table.find_or_insert(uniq, n_dev=nu)
        if mark is not None:
            mark.record(stream)
        htl.gather(table, slots, inv, out=out)
        return uniq, inv, nu, slots, status

    T3, _, _ = _timed(torch, args, three_calls, restore)
    T, wall, (uniq, inv, nu, slots, status) = _timed(torch, args, step, restore)
    ms = float(T.step_ms().mean())
    g_ms = float(T.kernel_ms().mean())
    U = int(nu.item())
    hits, misses = _statuses(htl, status, U)
    row = w.dim * (4 if w.dtype == "f32" else 2)
    path_bytes, gather_bytes = _lookup_bytes(n, U, hits, misses, row)
    ms3, g3 = float(T3.step_ms().mean()), float(T3.kernel_ms().mean())
    found = (status[:U] == htl.FOUND)[inv.long()].float().mean().item()
    config = {"workload": w.name, "ids_per_step": n, "zipf_a": w.meta.get("zipf_a"),
              "key_universe_log2": w.meta.get("universe_log2"), "table_slots_log2": w.capacity_log2,
              "prefilled_keys": 0 if w.prefill is None else int(w.prefill.size), "dim": w.dim,
              "row_dtype": w.dtype, "parallelism": "single GPU"}
    path = {"unique": U, "hits": hits, "misses": misses, "hit_rate_per_id": round(found, 4),
            "algorithmic_bytes": path_bytes,
            "achieved_gbs": round(path_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(path_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_median": round(float(np.median(T.step_ms())), 4),
            "wall_ms_per_step_incl_restore": round(wall / args.steps * 1e3, 4),
            "implementation": "emb_lookup_slots (dedup_unique_inverse + ht_find_or_insert, each ID's slot "
                              "composed per tile after the insert) + emb_gather_pool over the per-ID slots",
            "three_calls": {"ms_per_step": round(ms3, 4), "gather_ms": round(g3, 4),
                            "mkeys_s": round(n / (ms3 * 1e-3) / 1e6, 1),
                            "implementation": "dedup_unique_inverse + ht_find_or_insert + "
                                              "emb_gather_pool(slots, inverse)"},
            "timing": "HIP events around the whole step on the launch stream; table keys "
                      "restored by a D2D copy between steps, outside the events"}
    if w.name == "single_large_table" and not args.no_pcie:
        path["pcie_inclusive"] = _pcie_inclusive(torch, htl, table, w, dev, out, restore)
    traffic = _measured_traffic(w.name) if w.name == "single_large_table" else None
    res = _result(args, n / (ms * 1e-3) / 1e6, ms, config,
                  "int64 keys, " + ("fp32" if w.dtype == "f32" else "bf16") + " rows", path,
                  _roofline("k_gather (emb_gather_pool: per-ID rows)", gather_bytes, g_ms, traffic))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline_lookup(w, args.cpu_sample)
    return res


def run_pooled(args, torch, htl, workloads, dev):
    w = workloads.merged_tables()
    warm = workloads.merged_tables(seed=1)
    n, nb = w.keys.size, w.nbags
    keys = torch.from_numpy(w.keys).to(dev)
    offsets = torch.from_numpy(w.offsets).to(dev)
    table = htl.Table(w.capacity_log2, w.dim, w.dtype)
    wk = torch.from_numpy(warm.keys).to(dev)             # a previous batch populates the table (untimed)
    u0, _, nu0 = htl.dedup_unique_inverse(wk)
    table.find_or_insert(u0, n_dev=nu0)
    del wk, u0
    saved_keys = htl.table_keys(table).clone()
    view = table.view()
    stream = torch.cuda.current_stream()
    out = torch.empty((nb, w.dim), dtype=torch.bfloat16, device=dev)

    def restore():
        htl._binding.copy_to_device_ptr(view.keys, saved_keys)

    bufs = _lookup_bufs(torch, n, dev)

    def step(mark):
        # emb_lookup_slots, then bag sums over the per-ID slots
        uniq, inv, nu, slots, status, ids = htl.lookup_slots(table, keys, bufs=bufs)
        if mark is not None:
            mark.record(stream)
        htl.gather_pool(table, ids, None, offsets, out_dtype="bf16", out=out)
        return uniq, inv, nu, slots, status

    def three_calls(mark):
        uniq, inv, nu = htl.dedup_unique_inverse(keys)
        slots, status = table.find_or_insert(uniq, n_dev=nu)
        if mark is not None:
            mark.record(stream)
        htl.gather_pool(table, slots, inv, offsets, out_dtype="bf16", out=out)
        return uniq, inv, nu, slots, status

    T3, _, _ = _timed(torch, args, three_calls, restore)
    T, wall, (uniq, inv, nu, slots, status) = _timed(torch, args, step, restore)
    ms, p_ms = float(T.step_ms().mean()), float(T.kernel_ms().mean())
    ms3, p3 = float(T3.step_ms().mean()), float(T3.kernel_ms().mean())
    U = int(nu.item())
    hits, misses = _statuses(htl, status, U)
    row = w.dim * 2
    # per ID: key 8 + inverse 4 + 4; per bag: offsets 4 + pooled row; per unique: 33 + a row read
    # (hits) or a key claim and a row write (misses)
    path_bytes = n * 16 + nb * (4 + row) + U * 33 + hits * row + misses * (8 + row)
    # pooling over the per-ID slots: per ID its slot, per bag offsets and the pooled row, each unique row once
    pool_bytes = n * 4 + nb * (4 + row) + U * row
    config = {"workload": w.name, "ids_per_step": n, "bags": nb, "tables": w.meta["n_tables"],
              "zipf_a": w.meta["zipf_a"], "mean_bag": w.meta["mean_bag"], "table_slots_log2": w.capacity_log2,
              "dim": w.dim, "row_dtype": "bf16", "pooled_dtype": "bf16", "parallelism": "single GPU"}
    path = {"unique": U, "hits": hits, "misses": misses, "algorithmic_bytes": path_bytes,
            "achieved_gbs": round(path_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(path_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "wall_ms_per_step_incl_restore": round(wall / args.steps * 1e3, 4),
            "implementation": "emb_lookup_slots (dedup + find-or-insert + each ID's slot) + emb_gather_pool "
                              "(bags over the per-ID slots)",
            "three_calls": {"ms_per_step": round(ms3, 4), "pool_ms": round(p3, 4),
                            "mkeys_s": round(n / (ms3 * 1e-3) / 1e6, 1),
                            "implementation": "dedup_unique_inverse + ht_find_or_insert + "
                                              "emb_gather_pool(slots, inverse, offsets)"},
            "timing": "HIP events per step; table keys restored between steps outside the events"}
    res = _result(args, n / (ms * 1e-3) / 1e6, ms, config, "int64 keys, bf16 rows, fp32 accumulate", path,
                  _roofline("k_pool_team (emb_gather_pool with bags)", pool_bytes, p_ms,
                            _measured_traffic("merged_tables")))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline_pooled(w, warm)
    return res


# ----------------------------------------------------------------- backward
def run_backward(args, torch, htl, workloads, dev):
    w = workloads.backward(with_grad=False)
    n, dim = w.keys.size, w.dim
    keys = torch.from_numpy(w.keys).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1_000_003)
    grad = torch.randn((n, dim), generator=gen, dtype=torch.float32, device=dev)
    table = htl.Table(w.capacity_log2, dim, "f32", adam=True)
    # the forward (untimed): its dedup (unique, inverse) and slots are what the backward consumes
    uniq, inv, nu = htl.dedup_unique_inverse(keys)
    slots, status = table.find_or_insert(uniq, n_dev=nu)
    stream = torch.cuda.current_stream()
    g = torch.empty((n, dim), dtype=torch.float32, device=dev)
    state = {"t": 0}
    hp = (1e-3, 0.9, 0.999, 1e-8)

    def fused(mark):
        if mark is not None:
            mark.record(stream)
        state["t"] += 1
        htl.segment_sum_adam(table, slots, grad, inv, nu, n, *hp, state["t"])
        return nu

    def two_calls(mark):
        htl.segment_sum(grad, inv, nu, u_max=n, out=g)
        if mark is not None:
            mark.record(stream)
        state["t"] += 1
        htl.rowwise_adam(table, slots, g, nu, *hp, state["t"])
        return nu

    T, wall, nq = _timed(torch, args, fused)
    ms = float(T.step_ms().mean())
    T2, _, _ = _timed(torch, args, two_calls)
    ms2 = float(T2.step_ms().mean())
    adam_ms = float(T2.kernel_ms().mean())
    seg_ms = ms2 - adam_ms
    U = int(nq.item())
    row = dim * 4
    # fused: per ID inverse 4 + gradient row; per unique slot 4 + theta, m, v read and written
    fused_bytes = n * (4 + row) + U * (4 + 6 * row)
    # two calls: the summed rows are written and read back in addition
    two_bytes = fused_bytes + 2 * U * row
    seg_bytes = n * (4 + row) + U * row
    config = {"workload": w.name, "ids_per_step": n, "zipf_a": w.meta["zipf_a"],
              "table_slots_log2": w.capacity_log2, "dim": dim, "grad_dtype": "fp32",
              "optimizer": "row-wise Adam lr=1e-3 b1=0.9 b2=0.999 eps=1e-8", "parallelism": "single GPU"}
    path = {"unique": U, "algorithmic_bytes": fused_bytes,
            "achieved_gbs": round(fused_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(fused_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
            "implementation": "emb_grad_segment_sum_adam (segment-sum with Adam applied per finished row) "
                              "over the forward's dedup",
            "two_calls": {"ms_per_step": round(ms2, 4), "segment_sum_ms": round(seg_ms, 4),
                          "adam_ms": round(adam_ms, 4), "algorithmic_bytes": two_bytes,
                          "segment_sum_achieved_gbs": round(seg_bytes / (seg_ms * 1e-3) / 1e9, 1),
                          "implementation": "emb_grad_segment_sum + emb_rowwise_adam"},
            "grad": "torch.randn on the GPU, seeded generator (1000003)",
            "timing": "HIP events per step; the forward's dedup and find-or-insert run once, untimed; "
                      "Adam's step counter advances"}
    res = _result(args, n / (ms * 1e-3) / 1e6, ms, config, "fp32 gradients and rows", path,
                  _roofline("emb_grad_segment_sum_adam (fused backward)", fused_bytes, ms,
                            _measured_traffic("backward")))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline_backward(w, grad[:1 << 22].cpu().numpy())
    return res


# ------------------------------------------------------------------- online
def run_online(args, torch, htl, workloads, dev):
    spec = workloads.DynamicOnlineSpec()
    steps = args.warmup + args.steps
    use_log = not args.no_access_log
    table = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True, growable=args.growable,
                      access_log=use_log)
    stream = torch.cuda.current_stream()
    out = torch.empty((spec.n, spec.dim), dtype=torch.bfloat16, device=dev)
    log_served = 0
    bufs = _lookup_bufs(torch, spec.n, dev)
    fwd, lru, ers, gat = [], [], [], []
    U_last = 0
    gen = workloads.DynamicOnlineStream(spec, steps)
    hold = _GpuHold(torch, stream)
    for s in range(steps):
        keys = torch.from_numpy(gen.keys(s)).to(dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        torch.cuda.synchronize()
        hold(4.0)                       # the host enqueues forward + LRU behind it
        e[0].record(stream)
        uniq, inv, nu, slots, status, ids = htl.lookup_slots(table, keys, step=s, bufs=bufs)
        e[5].record(stream)
        htl.gather(table, ids, None, out=out)
        e[1].record(stream)
        victims, nv = table.lru_select(spec.evict_num, spec.evict_den)
        e[2].record(stream)
        k = int(nv.item())                                # the host needs k to size the erase
        hold(1.0)
        e[3].record(stream)
        table.erase(victims[:k])
        e[4].record(stream)
        torch.cuda.synchronize()
        if s >= args.warmup:
            fwd.append(e[0].elapsed_time(e[1]))
            lru.append(e[1].elapsed_time(e[2]))
            ers.append(e[3].elapsed_time(e[4]))
            gat.append(e[5].elapsed_time(e[1]))
            U_last = int(nu.item())
            if use_log:       # outside the timed events: did the log serve this step's choice?
                log_served += int(table.access_log_state()[0].item())
        print(f"online step {s} done", file=sys.stderr, flush=True)
    ms = float(np.mean(fwd))
    M = 1 << spec.capacity_log2
    row = spec.dim * 2
    resize = None
    if args.growable:
        # one capacity doubling after the timed steps: rehash of the key index only
        live = int(table.scan()[3].item())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        table.resize(spec.capacity_log2 + 1)
        b.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        M2 = 2 * M
        rbytes = M * (8 + 4) + live * (8 + 4) + M2 * 8 + M * 4
        resize = {"from_slots_log2": spec.capacity_log2, "to_slots_log2": spec.capacity_log2 + 1,
                  "live_keys": live, "wall_ms": round(wall, 3),
                  "algorithmic_bytes": rbytes,
                  "rows_moved": 0,
                  "what": "map row space for 2^28 handles, new index, rehash of the live keys with their handles, "
                          "free of the old index (the call synchronises the stream)"}
    fwd_bytes = spec.n * (16 + row) + U_last * (33 + row)
    gather_bytes = spec.n * (4 + row) + U_last * row
    live_now = int(table.scan()[3].item())
    # the scan reads last_seen of every slot (dead slots are marked there)
    # and writes then reads back each live slot's (last_seen, slot); with
    # the access log the selection reads only the ring entries of the oldest
    # steps (a window the device chooses), so no fixed byte count applies
    lru_bytes = M * 4 + live_now * 8 * 2
    config = {"workload": "dynamic_online", "ids_per_step": spec.n, "window": spec.window,
              "new_ids_per_step": spec.delta, "zipf_a": spec.zipf_a, "table_slots_log2": spec.capacity_log2,
              "dim": spec.dim, "row_dtype": "bf16", "evict_fraction": f"{spec.evict_num}/{spec.evict_den}",
              "access_log": use_log, "parallelism": "single GPU"}
    ckpt = None
    if args.checkpoint:
        ckpt = _time_checkpoint(torch, htl, table, spec, stream)
    path = {"unique_last_step": U_last, "forward_ms": round(ms, 4),
            "lru_select_ms": round(float(np.mean(lru)), 4), "erase_ms": round(float(np.mean(ers)), 4),
            "live_keys": live_now,
            "lru_select_path": ("access log (cut step from per-step live counts, candidates from the ring "
                                "entries of the oldest steps)" if use_log else "last_seen scan"),
            "lru_select_log_served_steps": f"{log_served}/{args.steps}" if use_log else None,
            "lru_select_roofline": None if use_log else _roofline(
                "ht_lru_select (last_seen scan + radix select, all its kernels)", lru_bytes, float(np.mean(lru))),
            "forward_algorithmic_bytes": fwd_bytes,
            "table": "growable (row handles, mapped row space)" if args.growable else "fixed",
            "resize": resize,
            "checkpoint": ckpt,
            "implementation": "emb_lookup_slots(step) + gather over the per-ID slots, then ht_lru_select + "
                              "ht_erase",
            "timing": f"per-step HIP events over steps {args.warmup}..{steps - 1} of the drifting stream "
                      "(the warm-up steps fill the table); a GPU spin kernel (torch.cuda._sleep) holds the "
                      "stream while the host enqueues each phase, so the events time GPU work, not launch "
                      "overhead; value = forward IDs/s"}
    res = _result(args, spec.n / (ms * 1e-3) / 1e6, ms, config, "int64 keys, bf16 rows", path,
                  _roofline("k_gather (forward per-ID rows, bf16)", gather_bytes, float(np.mean(gat)),
                            None if args.growable else _measured_traffic("dynamic_online")))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline_online(workloads, spec)
    return res


def _pcie_inclusive(torch, htl, table, w, dev, out, restore, steps=12):
    """Keys arriving in pinned host memory each step: one stream (H2D copy,
    then the lookup) against two (the next batch's copy on a second stream
    while the current batch is looked up).  Wall time over `steps` steps;
    the table-key restore between steps runs in both."""
    n = w.keys.size
    host = torch.from_numpy(w.keys).pin_memory()
    bufs = [torch.empty(n, dtype=torch.int64, device=dev) for _ in range(2)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    lbufs = _lookup_bufs(torch, n, dev)

    def lookup(k):
        _, _, _, _, _, ids = htl.lookup_slots(table, k, bufs=lbufs)
        htl.gather(table, ids, None, out=out)

    # the H2D rate alone
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(main)
    for _ in range(4):
        bufs[0].copy_(host, non_blocking=True)
    b.record(main)
    torch.cuda.synchronize()
    h2d_gbs = 4 * n * 8 / (a.elapsed_time(b) * 1e-3) / 1e9

    def one_stream(k):
        for _ in range(k):
            bufs[0].copy_(host, non_blocking=True)
            lookup(bufs[0])
            restore()

    def two_streams(k):
        E = lambda: torch.cuda.Event()  # noqa: E731
        copied, used = [E(), E()], [None, None]
        with torch.cuda.stream(side):
            bufs[0].copy_(host, non_blocking=True)
            copied[0].record(side)
        for i in range(k):
            cur, nxt = i % 2, 1 - i % 2
            if i + 1 < k:
                with torch.cuda.stream(side):
                    if used[nxt] is not None:
                        side.wait_event(used[nxt])
                    bufs[nxt].copy_(host, non_blocking=True)
                    copied[nxt].record(side)
            main.wait_event(copied[cur])
            lookup(bufs[cur])
            used[cur] = E()
            used[cur].record(main)
            restore()

    def wall(f):
        f(2)                                   # warm-up: streams, events, workspaces
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        f(steps)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    seq = wall(one_stream)
    ovl = wall(two_streams)
    return {"h2d_gbs": round(h2d_gbs, 1),
            "one_stream_mkeys_s": round(steps * n / seq / 1e6, 1),
            "two_streams_mkeys_s": round(steps * n / ovl / 1e6, 1),
            "what": "keys copied from pinned host memory every step (32 MiB); wall time over "
                    f"{steps} steps including the table-key restore; not the headline value"}


def _time_checkpoint(torch, htl, table, spec, stream, chunk=1 << 24):
    """Export the whole table range by range into reused device buffers
    (events, stream held while each call is enqueued), copy the live entries
    into pinned host memory, and import them into a fresh table of the same
    shape (events)."""
    M = table.capacity
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    hold = _GpuHold(torch, stream)
    bufs = table.export_buffers(chunk)
    host_parts, exp_ms, d2h_ms = [], 0.0, 0.0
    for b in range(0, M, chunk):
        a, c = E(), E()
        torch.cuda.synchronize()
        hold(1.0)
        a.record(stream)
        d = table.export(b, min(b + chunk, M), bufs=bufs)
        c.record(stream)
        n = int(d.pop("n").item())
        exp_ms += a.elapsed_time(c)
        part = {}
        a2, c2 = E(), E()
        a2.record(stream)
        for k, v in d.items():
            v = v[:n].view(torch.int16) if v.dtype == torch.bfloat16 else v[:n]
            h = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
            h.copy_(v, non_blocking=True)
            part[k] = h
        c2.record(stream)
        torch.cuda.synchronize()
        d2h_ms += a2.elapsed_time(c2)
        host_parts.append(part)
    live = sum(int(p["keys"].shape[0]) for p in host_parts)
    del bufs
    fresh = htl.Table(spec.capacity_log2, spec.dim, "bf16", last_seen=True)
    keys = torch.cat([p["keys"] for p in host_parts]).to(stream.device)
    rows = torch.cat([p["rows"] for p in host_parts]).to(stream.device).view(torch.bfloat16)
    ls = torch.cat([p["last_seen"] for p in host_parts]).to(stream.device)
    a, c = E(), E()
    torch.cuda.synchronize()
    hold(1.0)
    a.record(stream)
    st = fresh.import_(keys, rows, ls)
    c.record(stream)
    torch.cuda.synchronize()
    imp_ms = a.elapsed_time(c)
    ok = bool((st == htl.INSERTED).all().item())
    fresh.close()
    entry = 8 + spec.dim * 2 + 4
    return {"live_entries": live, "entry_bytes": entry,
            "export_ms": round(exp_ms, 3), "export_calls": M // chunk,
            "export_gbs": round((M * 8 + live * (entry + 4)) / (exp_ms * 1e-3) / 1e9, 1),
            "d2h_ms": round(d2h_ms, 3), "d2h_gbs": round(live * entry / (d2h_ms * 1e-3) / 1e9, 1),
            "import_ms": round(imp_ms, 3), "import_all_inserted": ok,
            "what": "ht_export over 2^24-slot ranges of the 2^27-slot table (the key array scanned, live "
                    "entries written), copy of the live entries to pinned host memory, ht_import into an "
                    "empty table"}


class _GpuHold:
    """Keeps the stream busy for about `ms` milliseconds (torch.cuda._sleep,
    calibrated once), so that work the host enqueues meanwhile then runs back
    to back and events around it time the GPU, not the Python launches."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        cyc = 1 << 20
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        torch.cuda._sleep(cyc)
        b.record(stream)
        torch.cuda.synchronize()
        self.cycles_per_ms = cyc / max(a.elapsed_time(b), 1e-3)

    def __call__(self, ms):
        self.torch.cuda._sleep(int(self.cycles_per_ms * ms))


# -------------------------------------------------------------- references
def _copy_reference(torch, htl, dev, nbytes=1 << 30, reps=5):
    """Achievable streaming bandwidth: a 1 GiB device-to-device copy (read +
    write) by the library's copy probe kernel, and by the runtime's copy."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    stream = torch.cuda.current_stream()

    def best_ms(copy):
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            copy()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        return best

    probe = 2 * nbytes / (best_ms(lambda: htl.copy_probe(src, dst)) * 1e-3) / 1e9
    assert torch.equal(src[:1 << 20], dst[:1 << 20]) and torch.equal(src[-(1 << 20):], dst[-(1 << 20):])
    runtime = 2 * nbytes / (best_ms(lambda: htl._binding.copy_to_device_ptr(dst.data_ptr(), src)) * 1e-3) / 1e9
    return {"kind": "htl_copy_probe (16 B per lane, full grid), 1 GiB, best of 5", "gbs": round(probe, 1),
            "frac_of_peak": round(probe / HBM_PEAK_GBS, 4), "runtime_memcpy_gbs": round(runtime, 1)}


def _cpu_baseline_lookup(w, sample, reps=6):
    """The oracle timed on the host (single thread) on the first `sample` IDs,
    `reps` passes; between passes the keys a pass inserted are erased
    (untimed), so every pass sees the pre-filled table."""
    import oracle
    m = min(sample, w.keys.size)
    keys = np.ascontiguousarray(w.keys[:m])
    tab = oracle.Table(1 << w.capacity_log2, w.dim, oracle.F32 if w.dtype == "f32" else oracle.BF16)
    if w.prefill is not None:
        tab.find_or_insert(w.prefill)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        uniq, inv = oracle.dedup(keys)
        st = tab.find_or_insert(uniq)
        tab.gather(keys)
        times.append(time.perf_counter() - t0)
        tab.erase(uniq[st == oracle.INSERTED])
    dt = float(np.median(times))
    return {"value": round(m / dt / 1e6, 3), "unit": "Mkeys/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m} IDs of the same batch, dedup+find_or_insert+gather, median of {reps} passes "
                      f"({sum(times):.1f} s timed in all); the table is pre-filled untimed and the keys a pass "
                      "inserts are erased untimed before the next", "host_cpus": os.cpu_count()}


def _cpu_baseline_pooled(w, warm, samples=16384, reps=3):
    """The oracle on the bags of the first `samples` samples (sample-major, so
    a prefix of the batch): dedup + find-or-insert + sum-pooling, `reps`
    passes on a table warmed (untimed) by the same samples of the earlier
    batch; the keys a pass inserts are erased untimed before the next."""
    import oracle
    nb = min(samples * w.meta["n_tables"], w.nbags)
    keys = np.ascontiguousarray(w.keys[:w.offsets[nb]])
    offsets = np.ascontiguousarray(w.offsets[:nb + 1])
    wb = min(nb, warm.nbags)
    tab = oracle.Table(1 << w.capacity_log2, w.dim, oracle.BF16)
    tab.find_or_insert(np.unique(warm.keys[:warm.offsets[wb]]))
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        uniq, _ = oracle.dedup(keys)
        st = tab.find_or_insert(uniq)
        tab.gather_pool(keys, offsets, oracle.BF16)
        times.append(time.perf_counter() - t0)
        tab.erase(uniq[st == oracle.INSERTED])
    dt = float(np.median(times))
    return {"value": round(keys.size / dt / 1e6, 3), "unit": "Mkeys/s", "cores": 1, "kind": "oracle",
            "sample": f"the {nb} bags of the first {nb // w.meta['n_tables']} samples ({keys.size} IDs), "
                      f"dedup+find_or_insert+sum-pool, median of {reps} passes ({sum(times):.1f} s timed in all); "
                      "the table is warmed untimed by the same samples of the earlier batch",
            "host_cpus": os.cpu_count()}


def _cpu_baseline_backward(w, grad_host, reps=6):
    """The oracle on the first len(grad_host) IDs: segment-sum (fp64) and the
    row-wise Adam step on the rows hit, `reps` passes; the dedup and the
    inserts of the keys run untimed, as the forward does on the GPU."""
    import oracle
    m = grad_host.shape[0]
    keys = np.ascontiguousarray(w.keys[:m])
    uniq, inv = oracle.dedup(keys)
    tab = oracle.Table(1 << w.capacity_log2, w.dim, oracle.F32, adam=True)
    tab.find_or_insert(uniq)
    times = []
    for t in range(1, reps + 1):
        t0 = time.perf_counter()
        s, _ = oracle.segment_sum(grad_host, inv, uniq.size, want_abs=False)
        tab.adam(uniq, s.astype(np.float32), step=t)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": round(m / dt / 1e6, 3), "unit": "Mkeys/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m} IDs and their gradient rows ({uniq.size} unique keys), segment-sum (fp64) + "
                      f"row-wise Adam, median of {reps} passes ({sum(times):.1f} s timed in all)",
            "host_cpus": os.cpu_count()}


def _cpu_baseline_online(workloads, spec, steps=6, m=1 << 22):
    """The oracle on the first `m` IDs of each of the first `steps` steps of
    the drifting stream: per step, dedup + find-or-insert + gather (timed as
    the forward), then the least-recently-used choice and its erase (timed
    apart); the median over the steps after the first."""
    import oracle
    gen = workloads.DynamicOnlineStream(spec, steps)
    tab = oracle.Table(1 << spec.capacity_log2, spec.dim, oracle.BF16)
    fwd, lru = [], []
    for s in range(steps):
        keys = np.ascontiguousarray(gen.keys(s)[:m])
        t0 = time.perf_counter()
        uniq, _ = oracle.dedup(keys)
        tab.find_or_insert(uniq, step=s)
        tab.gather(keys)
        t1 = time.perf_counter()
        tab.erase(tab.lru_victims(spec.evict_num, spec.evict_den))
        t2 = time.perf_counter()
        fwd.append(t1 - t0)
        lru.append(t2 - t1)
    dt = float(np.median(fwd[1:]))
    return {"value": round(m / dt / 1e6, 3), "unit": "Mkeys/s", "cores": 1, "kind": "oracle",
            "lru_choice_and_erase_ms": round(float(np.median(lru[1:])) * 1e3, 1),
            "sample": f"first {m} IDs of each of the first {steps} steps: forward (dedup+find_or_insert+gather) "
                      f"and, timed apart, the LRU choice of 5% of the live keys and their erase; median over "
                      f"steps 1..{steps - 1} ({sum(fwd) + sum(lru):.1f} s timed in all)",
            "host_cpus": os.cpu_count()}


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
    runner = {"single_large_table": run_lookup, "tiny": run_lookup, "merged_tables": run_pooled,
              "backward": run_backward, "dynamic_online": run_online}[args.workload]
    result = runner(args, torch, htl, workloads, dev)
    result["copy_reference"] = ref = _copy_reference(torch, htl, dev)
    # the dominant kernel's algorithmic rate against the measured copy rate
    result["roofline"]["frac_of_copy_probe"] = round(result["roofline"]["achieved"] / ref["gbs"], 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
