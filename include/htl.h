/*
 * htl.h -- C ABI of the MI355X (gfx950) sparse-embedding lookup library.
 *
 * The library implements the embedding hot path of a generative-recommendation
 * training system: feature-ID deduplication, a dynamic open-addressing hash
 * embedding table (find-or-insert, erase, scan), row gather with optional
 * sum-pooling over multi-hot bags, and the backward gradient segment-sum with
 * a row-wise Adam update.  Sources for each operation are cited below:
 *
 *   [MTGenRec] MTGenRec: An Efficient Distributed Training System for
 *              Generative Recommendation Models in Meituan (arXiv 2505.12663).
 *   [MTGR]     MTGR: Industrial-Scale Generative Recommendation Framework in
 *              Meituan (arXiv 2505.18654).
 *   [TF-PS]    Deep Customization of TensorFlow for Large-Scale Sparse Training
 *              at Meituan (technical article).
 *
 * Conventions for every call:
 *   - Pointers named in a signature are DEVICE pointers unless stated
 *     otherwise; the caller owns them (inputs, outputs and workspaces).  The
 *     library owns the table's storage.  No pointer is retained after return.
 *   - Every call that takes a stream only enqueues work on it (asynchronous).
 *     Calls on one table must be ordered on one stream, or synchronised by
 *     the caller.  Concurrent calls on one table race.
 *   - Sizes that depend on the data (unique count, live count, victim count)
 *     are produced on the device as int64 values; host-visible sizes passed
 *     in are upper bounds.
 *   - Argument errors are reported synchronously as HTL_ERR_INVALID before
 *     anything is enqueued; launch failures as HTL_ERR_DEVICE; allocation
 *     failures as HTL_ERR_NOMEM.  htl_last_error() then returns a message
 *     (thread-local, valid until the next call on the same thread).
 *     Data-dependent outcomes (full table, reserved key, key not found) are
 *     per-key status codes, never errors.
 *   - Device pointers must be aligned to their element size; row buffers
 *     (outputs of the gather, gradients) to 16 bytes.
 */
#ifndef HTL_H_
#define HTL_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct htl_table htl_table; /* opaque; created and owned by the library */

typedef enum {
    HTL_OK = 0,
    HTL_ERR_INVALID = 1, /* bad argument; nothing was enqueued */
    HTL_ERR_NOMEM = 2,   /* device allocation failed */
    HTL_ERR_DEVICE = 3   /* HIP runtime or launch error */
} htl_status;

/* The last enumerator gives the type the whole int range, so a value out of
 * range passed from C is a checked argument error, not undefined behaviour
 * in the library's C++ (the same for htl_dedup_path below). */
typedef enum { HTL_F32 = 0, HTL_BF16 = 1, HTL_DTYPE_RANGE_ = 0x7FFFFFFF } htl_dtype;

/* Per-key status of ht_find_or_insert (uint8 each). */
enum { HT_FOUND = 0, HT_INSERTED = 1, HT_FULL = 2, HT_RESERVED = 3 };
/* Per-key status of ht_erase (uint8 each). */
enum { HT_NOT_FOUND = 0, HT_ERASED = 1 };
/* ht_create flags. */
enum { HT_META_LAST_SEEN = 1u, HT_ADAM_STATE = 2u, HT_GROWABLE = 4u, HT_META_ACCESS_LOG = 8u };

/* Key values the table keeps for itself (slot markers). */
#define HT_EMPTY_KEY ((int64_t)-1)
#define HT_TOMBSTONE_KEY ((int64_t)-2)
/* Largest supported capacity_log2 (2^31 slots: slot indices are int32). */
#define HT_MAX_CAPACITY_LOG2 31

/* ------------------------------------------------------------------ table --
 * ht_create -- allocate an empty dynamic embedding table.
 * [MTGenRec] Abstract and Figure 5: embeddings kept in a table indexed by a
 * hash of the key, in place of fixed-size tables; [MTGR] section 5
 * "Embedding Management": each key leads to its embedding row and its
 * per-key metadata.  Theorem 1 of [MTGenRec] fixes the shape: M =
 * 2^capacity_log2 slots probed with an odd step.
 *   capacity_log2  1..HT_MAX_CAPACITY_LOG2; M = 2^capacity_log2 slots.
 *   dim            row length, 1..65536 elements.
 *   dtype          HTL_F32 or HTL_BF16 row elements.
 *   init_seed      seed of the closed-form initial row of every new key: the
 *                  row is a function of (key, init_seed) only.
 *   flags          HT_META_LAST_SEEN: keep a uint32 last_seen per slot;
 *                  HT_ADAM_STATE: keep fp32 Adam moments m, v (needs HTL_F32);
 *                  HT_GROWABLE: a table that ht_resize can grow (below);
 *                  HT_META_ACCESS_LOG: keep an access log for eviction
 *                  (needs HT_META_LAST_SEEN, capacity_log2 <= 30; below).
 *   stream         the table is cleared (all slots EMPTY) on this stream.
 * Storage, all on the current device: keys int64[M]; rows dtype[M][dim];
 * last_seen uint32[M]; m, v float[M][dim].  *t receives the handle.
 *
 * Growable tables ([MTGR] section 5: each key leads to its row and
 * metadata, and the table grows by copying what indexes the keys while the
 * embedding rows stay where they are): the key
 * index (keys int64[M], a row handle int32[M] and last_seen uint32[M] per
 * slot) is separate from the row space (rows, m, v indexed by row handle).
 * The row space is a reserved virtual range of up to
 * 2^min(30, capacity_log2 + 8) rows, of which M are mapped; ht_resize maps
 * more and rehashes only the index.  In
 * such a table every "slot" that a call returns or takes (ht_find_or_insert,
 * ht_scan, emb_gather_pool, emb_rowwise_adam) is a row handle: stable for as
 * long as its key stays live, across resizes; the handle of an erased key is
 * reused by a later insert.  capacity_log2 <= 30 (the row handles are int32
 * and the reservation must fit).
 *
 * Access log ([MTGR] section 5: per-key metadata, and scanning only what is
 * needed; the eviction policy is this library's, see ht_lru_select).  Each
 * find-or-insert appends one 8-byte entry per key, (slot, step) for keys it
 * inserts or re-stamps, to a ring of max(2^12, M/4) entries, and keeps per
 * step the number of live keys whose last_seen is that step (a record per
 * step mod 2^12, with 32 partial counts of one cache line each: 16 MiB).  ht_lru_select then finds the cut
 * step from those counts and reads only the ring entries of the oldest
 * steps up to it, instead of the last_seen of all M slots; its result is
 * the same.  The log serves while steps never decrease from one
 * find-or-insert to the next, no key is inserted at a step during which an
 * erase ran, the live keys' last_seen span fewer than 2^12 steps and the
 * entries from the oldest live step on fit in the ring; ht_import and
 * ht_resize end it.  Once it stops serving, ht_lru_select scans last_seen
 * as on a table without the log, until ht_clear restarts the log empty or
 * ht_access_log_rebuild rebuilds it from the live keys.  Writing
 * keys or last_seen through ht_view also ends what the log can vouch for,
 * without the library knowing: do not, on a logged table.  Part of the
 * log's bookkeeping is kept by the host at each call (which of two head
 * words the call reads, the step order, the erase rule above), so the
 * find-or-insert and erase calls of a logged table must be enqueued call by
 * call, not replayed from a captured HIP graph.
 * Errors: INVALID for a bad size/flag combination or null t; NOMEM; DEVICE
 * if the device cannot map virtual memory (HT_GROWABLE only). */
htl_status ht_create(htl_table** t, int capacity_log2, int dim, htl_dtype dtype,
                     uint64_t init_seed, uint32_t flags, hipStream_t stream);

/* ht_destroy -- free the table (synchronises the device first).  Null is a no-op. */
htl_status ht_destroy(htl_table* t);

/* ht_clear -- mark every slot EMPTY again (rows, metadata are left as they
 * are; a growable table also takes back every row handle; an access log
 * restarts empty). */
htl_status ht_clear(htl_table* t, hipStream_t stream);

/* ht_resize -- grow a growable table to 2^new_capacity_log2 slots ([MTGR]
 * section 5: capacity expansion replicates the key storage, not the
 * embeddings).  Maps row space for the new capacity, builds a new key index
 * (every live key re-inserted with its row handle; tombstones are dropped),
 * then frees the old index.  Rows and Adam moments do not move, so every
 * row handle stays valid; last_seen moves with its key.  new_capacity_log2 may equal the current
 * one (a rehash that only drops tombstones).  Synchronises `stream` before it
 * frees the old index; allocates device memory (hipMalloc / hipMemMap).
 * Errors: INVALID if the table is not growable, or new_capacity_log2 is below
 * the current one or above the reservation (2^min(30, created + 8) slots);
 * NOMEM; DEVICE. */
htl_status ht_resize(htl_table* t, int new_capacity_log2, hipStream_t stream);

/* ht_find_or_insert -- look up keys, inserting the absent ones.
 * [MTGenRec] Abstract (real-time insertion), Theorem 1 (odd-step probing of a
 * power-of-two table visits every slot); [MTGR] section 5 (keys -> vectors and
 * metadata).  Probing walks buckets of min(16, M) consecutive slots with an
 * odd bucket step, so every slot is reachable (Theorem 1 at bucket level) and
 * HT_FULL is only reported when no slot on the whole walk is free.
 *   keys     int64[n_max], device.  Precondition: the first n keys are
 *            pairwise distinct (dedup_unique_inverse produces such a list).
 *   n_max    host upper bound on the number of keys (sizes the launch).
 *   n_dev    nullable device int64: the actual count n <= n_max (e.g. the
 *            unique count written by dedup_unique_inverse); null means n_max.
 *   step     stamped into last_seen of FOUND and INSERTED keys (if kept);
 *            on a table that keeps last_seen, 0xFFFFFFFF is reserved (it
 *            marks slots with no live key) and is refused (HTL_ERR_INVALID).
 *   slots    int32[n_max] out: slot of each key (growable tables: its row
 *            handle), -1 for FULL and RESERVED.
 *   status   uint8[n_max] out: HT_FOUND, HT_INSERTED (row set to the closed-
 *            form initial row, Adam moments zeroed), HT_FULL, or HT_RESERVED
 *            (key equals HT_EMPTY_KEY or HT_TOMBSTONE_KEY).
 * Entries at index >= n are not written.  Erased slots (tombstones) are
 * reused by inserts.  A growable table hands out row handles with a count,
 * scan and assign pass (no shared counter) and keeps per-call temporaries
 * of 8 bytes per key, allocated on first use and grown when n_max grows. */
htl_status ht_find_or_insert(htl_table* t, const int64_t* keys, int64_t n_max,
                             const int64_t* n_dev, uint32_t step, int32_t* slots,
                             uint8_t* status, hipStream_t stream);

/* ht_erase -- delete keys ([MTGenRec] Abstract: real-time deletion).  A
 * deleted slot becomes a tombstone: lookups walk past it, inserts reuse it.
 *   keys    int64[n] device; duplicates allowed (one of them reports ERASED).
 *   status  uint8[n] out: HT_ERASED or HT_NOT_FOUND; nullable. */
htl_status ht_erase(htl_table* t, const int64_t* keys, int64_t n, uint8_t* status,
                    hipStream_t stream);

/* ht_scan -- compact listing of live slots ([MTGR] section 5, "compact key
 * scanning").  Writes, for each live slot in slot order, its key, its
 * last_seen (if kept) and its slot index (growable tables: its row handle).
 * Keeps per-call temporaries with the table (allocated on first use).
 *   keys       int64[M] out (nullable)    last_seen uint32[M] out (nullable)
 *   slots      int32[M] out (nullable)    n_live_dev int64 out: live count. */
htl_status ht_scan(const htl_table* t, int64_t* keys, uint32_t* last_seen, int32_t* slots,
                   int64_t* n_live_dev, hipStream_t stream);

/* ht_export -- checkpoint: the live entries of slots [slot_begin, slot_end),
 * written compactly in slot order ([MTGR] section 5, "compact key
 * scanning"), so that a table is saved range by range with bounded buffers.
 *   keys       int64[slot_end - slot_begin] out (nullable)
 *   rows       dtype[slot_end - slot_begin][dim] out (nullable; 16-byte
 *              aligned when a row is a multiple of 16 bytes)
 *   last_seen  uint32[...] out (nullable; the table must keep it)
 *   adam_m, adam_v  float[...][dim] out (nullable; the table must keep them)
 *   n_dev      int64 out: number of entries written.
 * Keeps per-call temporaries with the table (allocated on first use). */
htl_status ht_export(const htl_table* t, int64_t slot_begin, int64_t slot_end, int64_t* keys,
                     void* rows, uint32_t* last_seen, float* adam_m, float* adam_v,
                     int64_t* n_dev, hipStream_t stream);

/* ht_import -- restore: find-or-insert each key (as ht_find_or_insert with
 * step 0), then set the live ones' row, and where given their last_seen and
 * Adam moments, to the values passed (keys are distinct, as for
 * ht_find_or_insert).  An export followed by an import into an empty table
 * of the same dim and dtype reproduces every live key's state.
 *   keys int64[n]; rows dtype[n][dim]; last_seen uint32[n] (nullable);
 *   adam_m, adam_v float[n][dim] (both or neither);
 *   status uint8[n] out: as ht_find_or_insert (FULL / RESERVED keys are not
 *   written).  A last_seen of 0xFFFFFFFF (reserved, see ht_find_or_insert)
 *   is stored as 0xFFFFFFFE.  After an import with last_seen, eviction
 *   selections examine all four bytes of last_seen (the values are not
 *   known on the host). */
htl_status ht_import(htl_table* t, const int64_t* keys, int64_t n, const void* rows,
                     const uint32_t* last_seen, const float* adam_m, const float* adam_v,
                     uint8_t* status, hipStream_t stream);

/* ht_lru_select -- choose eviction victims for an online table: the
 * floor(live * num / den) live keys smallest by (last_seen, key), last_seen
 * compared as uint32 and keys as int64.  [MTGenRec] Abstract (deletions in
 * real time); [MTGR] section 5 (metadata per key, key scanning).  The pages
 * name no policy: least-recently-used with a key tie-break is this library's.
 * Needs HT_META_LAST_SEEN and capacity_log2 <= 30 (HTL_ERR_INVALID otherwise).
 *   victims        int64[victims_cap] out: the victim keys, unspecified order.
 *   n_victims_dev  int64 out: the number of victims k (also when k exceeds
 *                  victims_cap, in which case victims holds an arbitrary
 *                  subset of victims_cap of them).
 *   ws, ws_bytes   workspace of at least lru_workspace_bytes(t) bytes. */
size_t lru_workspace_bytes(const htl_table* t);
htl_status ht_lru_select(const htl_table* t, int64_t num, int64_t den, int64_t* victims,
                         int64_t victims_cap, int64_t* n_victims_dev, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* ht_rows -- read-only view of the table's embedding rows ([MTGR] section 5,
 * "Embedding Management": the table keeps, per key, an embedding vector and
 * metadata).  *rows receives the device address of dtype[R][dim], where R is
 * the capacity (rows indexed by slot) or, for a growable table, the rows
 * mapped so far (indexed by row handle); *row_bytes receives dim times the
 * element size.  The caller reads the rows of the slots / handles that
 * ht_find_or_insert or ht_scan returned; it must not write through the
 * pointer.  The pointer stays valid until ht_destroy (a growable table's row
 * space never moves: ht_resize maps more rows behind it).  Either output may
 * be null.  Errors: INVALID for a null table. */
htl_status ht_rows(const htl_table* t, const void** rows, int64_t* row_bytes);

/* htl_debug_build -- 1 if the library was built with -DHTL_DEBUG, else 0.
 * A debug build enqueues, after each find-or-insert, dedup and logged erase,
 * a kernel that checks the table's invariants on the device and records
 * violations as bits of a per-device flag word (it never stops a kernel):
 *   HTL_DEBUG_SLOT   a FOUND / INSERTED key is not in the slot returned
 *   HTL_DEBUG_DUP    a FOUND / INSERTED key occurs other than once on its walk
 *   HTL_DEBUG_WALK   a walk took more than M/16 buckets (Theorem 1 of [MTGenRec]
 *                    at bucket level: M/16 buckets reach every slot)
 *   HTL_DEBUG_FULL   a FULL key's walk holds a free slot or a copy of the key
 *   HTL_DEBUG_DEDUP  unique[inverse[i]] != keys[i], or n_unique out of [1, n]
 *   HTL_DEBUG_LOG    an access log's live count of a step is negative
 * htl_debug_flags -- synchronise the current device, write its flag word to
 * *flags_out and clear it (0 in a release build).  Errors: INVALID for a
 * null output; DEVICE. */
#define HTL_DEBUG_SLOT 1u
#define HTL_DEBUG_DUP 2u
#define HTL_DEBUG_WALK 4u
#define HTL_DEBUG_FULL 8u
#define HTL_DEBUG_DEDUP 16u
#define HTL_DEBUG_LOG 32u
int htl_debug_build(void);
htl_status htl_debug_flags(uint32_t* flags_out);

/* ht_access_log_rebuild -- rebuild a table's access log from its live keys
 * and their last_seen (after ht_import, ht_resize or an overflow ended it):
 * the live keys' entries go to the ring in step order and each step's count
 * is set, so that the log serves the next eviction choice again.  Reads
 * last_seen of every slot twice; allocates small temporaries and
 * synchronises `stream`.  Errors: INVALID for a null table, a table without
 * HT_META_ACCESS_LOG, or live keys whose last_seen span 4096 steps or more or
 * that outnumber the ring's entries (the log then stays off); NOMEM; DEVICE. */
htl_status ht_access_log_rebuild(htl_table* t, hipStream_t stream);

/* ht_access_log_state -- where a table's access log stands (see ht_create),
 * for tests and monitoring.  Writes int64[4] to out_dev on `stream`: [0] 1
 * if the log serves the next eviction choice, else 0; [1] its head and [2]
 * its tail (ring positions, unwrapped); [3] the oldest step that may still
 * have live keys.  Errors: INVALID for a null table or output, or a table
 * created without HT_META_ACCESS_LOG; DEVICE. */
htl_status ht_access_log_state(const htl_table* t, int64_t* out_dev, hipStream_t stream);

/* ht_view -- every storage array of the table, for checkpoint tooling,
 * tests and measurement.  Any output may be null.  rows is dtype[M][dim]; m,
 * v are null unless the table keeps Adam state; last_seen (per slot;
 * 0xFFFFFFFF at slots with no live key) is null unless it keeps metadata.  In
 * a growable table rows, m and v are indexed by row handle, and row_of_slot
 * (int32[M], valid at live slots) maps a slot to its handle; row_of_slot is
 * null for other tables (handle = slot).  The pointers are the table's own
 * storage: reading them is always safe; a caller that writes through them
 * (a benchmark restoring the key array between timed steps, say) takes over
 * the table's invariants -- keys distinct, EMPTY / TOMBSTONE markers, the
 * last_seen marker of dead slots -- and must keep them. */
typedef struct {
    int64_t capacity;
    int32_t dim;
    int32_t dtype;
    int64_t* keys;
    void* rows;
    uint32_t* last_seen;
    float* adam_m;
    float* adam_v;
    int32_t* row_of_slot;
} htl_view;
htl_status ht_view(const htl_table* t, htl_view* out);

/* ------------------------------------------------------------------ dedup --
 * dedup_unique_inverse -- feature-ID deduplication in two stages.
 * [MTGenRec] TL;DR (one of its four components: IDs are deduplicated in two
 * stages to speed up the embedding lookup) and table of contents section 6,
 * "Embedding Table Lookup Acceleration"; [MTGR] section 5 "Embedding Lookup":
 * the IDs stay unique both before and after the cross-device exchange.  On one device,
 * stage 1 dedups each tile of keys in on-chip memory (one copy per tile
 * leaves it, as one copy per sender leaves a device before the exchange), and
 * stage 2 dedups the tile survivors device-wide: for 2048 < n <= 2^23 by hash
 * bins, each deduplicated in on-chip memory by one workgroup (no device
 * atomics), for larger n through one device-wide set.
 *   keys          int64[n]; every 64-bit value is a valid key.
 *   unique        int64[n] out: the U distinct keys.  Order: unspecified
 *                 (hash-bin order for the binned stage 2, and within a bin
 *                 the order in which survivors arrive; with the set, the
 *                 tile order of the survivor whose insert won); a batch of
 *                 at most 2048 keys is deduplicated in one launch and comes
 *                 out in first-occurrence order.
 *   inverse       int32[n] out: unique[inverse[i]] == keys[i].
 *   n_unique_dev  int64 out: U.
 *   ws, ws_bytes  workspace of at least dedup_workspace_bytes(n) bytes,
 *                 256-byte aligned; contents on entry are ignored.
 * n must be below 2^30.  n == 0 writes U = 0. */
size_t dedup_workspace_bytes(int64_t n);
htl_status dedup_unique_inverse(const int64_t* keys, int64_t n, int64_t* unique,
                                int32_t* inverse, int64_t* n_unique_dev, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* dedup_unique_inverse_ordered -- the same, with `unique` in order of first
 * occurrence in keys: the output is a function of the input alone
 * (reproducible run to run).  Same arguments and workspace; slower (one more
 * atomic per unique key). */
htl_status dedup_unique_inverse_ordered(const int64_t* keys, int64_t n, int64_t* unique,
                                        int32_t* inverse, int64_t* n_unique_dev, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------- adaptive unique --
 * dedup_unique_inverse_adaptive -- dedup_unique_inverse whose second stage
 * is chosen per call by a heuristic, as the TensorFlow article's adaptive
 * Unique is ([TF-PS] section 3.6: a heuristic picks the Unique
 * implementation).  Same arguments, workspace (dedup_workspace_bytes(n)) and
 * results; unique is in an unspecified order.  The plan carries the
 * statistics of its previous calls: at the end of each call the device
 * writes n, the number of stage-1 survivors, U and the form it ran into
 * pinned host memory, and the next call reads them there without waiting
 * for the device (so the choice follows the stream one or a few batches
 * behind).  Forms (htl_dedup_path):
 *   HTL_DEDUP_ONE_TILE        n <= 2048: one workgroup, one launch;
 *   HTL_DEDUP_TWO_STAGE_BINS  per-tile dedup in LDS, then hash bins each
 *                             deduplicated in LDS (2048 < n <= 2^23);
 *   HTL_DEDUP_BINS_ONLY       the hash bins straight from the keys, no
 *                             stage 1 -- chosen while the duplicates stage 1
 *                             found in the plan's last measured batch (a
 *                             share d of its keys) are too few for any key
 *                             to overfill a bin: d n + n/2048 <= 3 n / P for
 *                             the P bins of the batch (every copy of a key
 *                             goes to one bin when stage 1 is skipped); a
 *                             batch run this way cannot measure d, so every
 *                             8th call of the plan runs both stages again;
 *   HTL_DEDUP_DEVICE_SET      per-tile dedup, then one device-wide set
 *                             (n > 2^23).
 * The first call of a plan, knowing nothing, takes the N-based default
 * (two-stage bins, or the form its size requires).  A plan belongs to one
 * device and one stream at a time; calls on it must be ordered.
 *
 * dedup_plan_create allocates the plan (a few bytes of pinned host memory);
 * dedup_plan_destroy synchronises the device, then frees it (null: no-op).
 * dedup_plan_stats returns what the device last reported (calls = 0 before
 * the first report lands); dedup_plan_choose the form the plan would take
 * for a batch of n keys now. */
typedef struct htl_dedup_plan htl_dedup_plan;
typedef enum {
    HTL_DEDUP_ONE_TILE = 0,
    HTL_DEDUP_TWO_STAGE_BINS = 1,
    HTL_DEDUP_BINS_ONLY = 2,
    HTL_DEDUP_DEVICE_SET = 3,
    HTL_DEDUP_PATH_RANGE_ = 0x7FFFFFFF
} htl_dedup_path;
typedef struct {
    int64_t calls;      /* calls whose statistics have landed */
    int64_t n;          /* keys of the last of them */
    int64_t survivors;  /* keys that left stage 1 (n when stage 1 was skipped) */
    int64_t n_unique;   /* U */
    int32_t path;       /* the htl_dedup_path it ran */
} htl_dedup_stats;
htl_status dedup_plan_create(htl_dedup_plan** plan);
htl_status dedup_plan_destroy(htl_dedup_plan* plan);
htl_status dedup_plan_stats(const htl_dedup_plan* plan, htl_dedup_stats* out);
int32_t dedup_plan_choose(const htl_dedup_plan* plan, int64_t n);
htl_status dedup_unique_inverse_adaptive(htl_dedup_plan* plan, const int64_t* keys, int64_t n, int64_t* unique,
                                         int32_t* inverse, int64_t* n_unique_dev, void* ws, size_t ws_bytes,
                                         hipStream_t stream);

/* dedup_unique_inverse_noalloc -- dedup_unique_inverse with no workspace
 * argument and no allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same kernels, arguments and results as dedup_unique_inverse;
 * the workspace is a fixed 64 MiB array in device memory that the library
 * carries (one per device, held from the library's first use on that
 * device until the process ends), so n is limited to
 * dedup_noalloc_max_keys() = 2^20 keys (HTL_ERR_INVALID beyond it, before
 * anything is enqueued).  The call allocates nothing: the array's device
 * address is looked up once per device, on the first call with that device
 * current (keys and outputs must live on the current device).  Every call on
 * one device shares that device's array, so calls that overlap on one
 * device -- on two streams, or from two threads without ordering -- race;
 * order them on one stream.  The array keeps the last call's contents; the
 * dedup reads nothing from it that it has not written in the same call. */
int64_t dedup_noalloc_max_keys(void);
htl_status dedup_unique_inverse_noalloc(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                        int64_t* n_unique_dev, hipStream_t stream);

/* ----------------------------------------------------------------- gather --
 * emb_gather_pool -- embedding row gather with optional bag sum-pooling.
 * [MTGenRec] TL;DR: the embedding lookup that the dynamic table and the
 * deduplication serve; [MTGR] section 5 "Other Optimizations" names table
 * lookup as the work of its dispatch stream.  Pooling over multi-hot bags is
 * this library's reading for bag-shaped features (the pages describe none).
 *   slots     int32[U]: table slot per unique key (from ht_find_or_insert);
 *             a negative slot stands for a zero row.
 *   inverse   nullable int32[n]: per-ID index into slots; null means the
 *             identity (ID i uses slots[i]).
 *   n         number of IDs.
 *   offsets   nullable int32[nbags + 1], non-decreasing, offsets[0] = 0,
 *             offsets[nbags] = n: CSR bags over the IDs.  Null = no pooling.
 *             The kernels clamp every bag to [0, n), so offsets that break
 *             this rule read no ID outside the n given (such a bag sums the
 *             IDs it keeps inside [0, n), possibly none).
 *   out_dtype HTL_F32 or HTL_BF16.  Without pooling it must equal the table's
 *             dtype, or be HTL_F32 for a bf16 table (exact widening).  With
 *             pooling, sums accumulate in fp32 and are rounded to bf16 to
 *             nearest even; an empty bag gives zeros.
 *   out       without pooling: out_dtype[n][dim] = copies of the rows;
 *             with pooling: out_dtype[nbags][dim]. */
htl_status emb_gather_pool(const htl_table* t, const int32_t* slots, const int32_t* inverse,
                           int64_t n, const int32_t* offsets, int64_t nbags,
                           htl_dtype out_dtype, void* out, hipStream_t stream);

/* ------------------------------------------------------------ one call --
 * emb_lookup_slots -- dedup_unique_inverse(keys), then
 * ht_find_or_insert(t, unique, n, n_unique_dev, step), and the slot of every
 * ID: id_slots[i] = slots[inverse[i]].  [MTGenRec] TL;DR and Figure 5 (IDs
 * deduplicated in two stages, then looked up in the dynamic hash table);
 * [MTGR] section 5 "Embedding Lookup".  unique, inverse, U, slots and status
 * are what the two calls write (unique in the same unspecified order), with
 * the same preconditions.  The dedup's last pass (the inverse, composed per
 * tile of IDs from the tile's distinct keys) runs after find-or-insert, so it
 * writes id_slots in the same pass, with one slot load per distinct key of a
 * tile instead of one per ID; a gather then reads one index per ID in
 * sequence: emb_gather_pool(t, id_slots, NULL, n, ...).
 *   keys, n        int64[n], 0 <= n < 2^30.
 *   step           as ht_find_or_insert.
 *   unique, inverse, n_unique_dev   as dedup_unique_inverse (unique int64[n]).
 *   slots, status  int32[n], uint8[n] out: as ht_find_or_insert on unique
 *                  (entries at index >= U are not written).
 *   id_slots       int32[n] out: the slot (growable tables: row handle) of
 *                  each ID's key, -1 for a RESERVED key.
 *   ws, ws_bytes   at least dedup_workspace_bytes(n) bytes, 256-byte
 *                  aligned; contents on entry are ignored.
 * Errors: every argument is checked before anything is enqueued
 * (HTL_ERR_INVALID); a growable table may allocate, as in ht_find_or_insert. */
htl_status emb_lookup_slots(htl_table* t, const int64_t* keys, int64_t n, uint32_t step, int64_t* unique,
                            int32_t* inverse, int64_t* n_unique_dev, int32_t* slots, uint8_t* status,
                            int32_t* id_slots, void* ws, size_t ws_bytes, hipStream_t stream);

/* emb_lookup -- the whole forward lookup in one call: emb_lookup_slots, then
 * emb_gather_pool(t, id_slots, NULL, n, offsets, nbags, out_dtype, out)
 * with id_slots kept in the workspace.  Every output equals what
 * dedup_unique_inverse, ht_find_or_insert and emb_gather_pool(t, slots,
 * inverse, ...) write.
 *   offsets, nbags, out_dtype, out  as emb_gather_pool.
 *   ws, ws_bytes   at least emb_lookup_workspace_bytes(n) bytes, 256-byte
 *                  aligned.
 * Other arguments and errors as emb_lookup_slots; the gather's arguments are
 * checked before anything is enqueued as well. */
size_t emb_lookup_workspace_bytes(int64_t n);
htl_status emb_lookup(htl_table* t, const int64_t* keys, int64_t n, uint32_t step, int64_t* unique,
                      int32_t* inverse, int64_t* n_unique_dev, int32_t* slots, uint8_t* status,
                      const int32_t* offsets, int64_t nbags, htl_dtype out_dtype, void* out, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------- backward --
 * emb_grad_segment_sum -- backward gradient dedup: out[u] = sum of grad[i]
 * over the IDs with inverse[i] == u, accumulated in fp32; summation order is
 * unspecified.  It is the backward of the deduplicated lookup: [MTGR]
 * section 5 "Embedding Lookup" keeps IDs unique around the exchange, and
 * [MTGenRec] TL;DR deduplicates IDs before the lookup, so every ID that
 * shares a unique key sends its gradient to that key's one row; the pages
 * describe no backward, and summing per unique key is the plain reading.
 *   grad          float[n][dim]; inverse int32[n] with values < U; entries
 *                 outside [0, U) contribute nowhere.  n < 2^31 - 1024,
 *                 1 <= dim <= 65536, 0 <= u_max <= n (HTL_ERR_INVALID
 *                 otherwise).
 *   n_unique_dev  device int64 U (nullable: then U = u_max); u_max host bound.
 *   out           float[u_max][dim]: rows 0..U-1 written, the rest untouched.
 *   ws, ws_bytes  at least segsum_workspace_bytes(n, u_max, dim) bytes,
 *                 256-byte aligned.  The size takes dim because segments
 *                 longer than one chunk of IDs leave a partial sum row
 *                 (dim floats) per chunk in the workspace. */
size_t segsum_workspace_bytes(int64_t n, int64_t u_max, int dim);
htl_status emb_grad_segment_sum(const float* grad, const int32_t* inverse, int64_t n,
                                const int64_t* n_unique_dev, int64_t u_max, int dim,
                                float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* emb_rowwise_adam -- Adam update of the rows hit by a batch.  [TF-PS]
 * section 3.2 (Adam with its beta terms kept per parameter server; here the
 * bias corrections are per-call scalars).  Per element, in fp32:
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g);
 *   theta -= lr * ((m / c1) / (sqrt(v / c2) + eps)),
 * c1 = 1 - b1^step, c2 = 1 - b2^step (computed in fp64 on the host).
 *   slots   int32[u_max]: slot of each unique key (negative: skipped).
 *   g       float[u_max][dim]: the summed gradient of each unique key.
 *   n_unique_dev nullable device int64 U <= u_max.  step >= 1.
 * Needs an HTL_F32 table with HT_ADAM_STATE. */
htl_status emb_rowwise_adam(htl_table* t, const int32_t* slots, const float* g, int64_t u_max,
                            const int64_t* n_unique_dev, float lr, float b1, float b2, float eps,
                            int64_t step, hipStream_t stream);

/* emb_grad_segment_sum_adam -- emb_grad_segment_sum and then emb_rowwise_adam
 * in one pass: each unique key's summed gradient is handed to Adam on its
 * table row as soon as it is complete, so the summed gradients are never
 * written to memory (the same arithmetic and results as the two calls, up to
 * the summation order, which is unspecified in both).  Backward of the
 * deduplicated lookup ([MTGenRec] TL;DR; [MTGR] section 5) with Adam as in
 * [TF-PS] section 3.2.
 *   t, slots      as emb_rowwise_adam; dim is the table's.
 *   grad, inverse, n, n_unique_dev, u_max  as emb_grad_segment_sum
 *                 (n < 2^31 - 1024, u_max <= n).
 *   ws, ws_bytes  at least segsum_adam_workspace_bytes(n, u_max, dim) bytes,
 *                 256-byte aligned.
 * Needs an HTL_F32 table with HT_ADAM_STATE; HTL_ERR_INVALID otherwise. */
size_t segsum_adam_workspace_bytes(int64_t n, int64_t u_max, int dim);
htl_status emb_grad_segment_sum_adam(htl_table* t, const int32_t* slots, const float* grad,
                                     const int32_t* inverse, int64_t n, const int64_t* n_unique_dev,
                                     int64_t u_max, float lr, float b1, float b2, float eps,
                                     int64_t step, void* ws, size_t ws_bytes, hipStream_t stream);

/* htl_copy_probe -- a plain streaming device-to-device copy (one 16-byte
 * vector per thread, full grid), the achievable-bandwidth reference against
 * which the lookup kernels' HBM rates are read.  A measurement aid, not a
 * step of the lookup path (the pages define no such operation).
 *   src, dst  device, 16-byte aligned, not overlapping; bytes a multiple of
 *             16 (HTL_ERR_INVALID otherwise).  Enqueued on `stream`. */
htl_status htl_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* htl_last_error -- message of the last failed call on this thread ("" if none). */
const char* htl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HTL_H_ */
