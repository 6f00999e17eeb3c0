// Dynamic open-addressing embedding table: create/clear/destroy/resize,
// find-or-insert, erase, compact scan, export / import (checkpoint).
//
// MTGenRec (arXiv 2505.12663): Abstract and Figure 5 (embeddings held in a
// table indexed by a hash of the key, in place of fixed-size tables, so that
// they can be added and removed while training runs), Theorem 1 (in a table of 2^n slots the walk
// h_t = h_0 + t*S mod 2^n visits every slot iff S is odd).  MTGR (arXiv
// 2505.18654) section 5, "Embedding Management": each key leads to its
// embedding row and its metadata, and live keys can be scanned compactly.
//
// Layout in HBM: keys int64[M] (EMPTY = -1, TOMBSTONE = -2), rows
// dtype[M][dim] indexed by slot, optional last_seen uint32[M], optional Adam
// moments float[M][dim].
//
// Growable tables (MTGR section 5: capacity grows by copying the key
// storage, not the embeddings) add a row handle int32[M] per slot; rows and
// the moments are indexed by handle and live in a reserved virtual range
// that grows by mapping physical memory at its end (hipMemAddressReserve /
// hipMemCreate / hipMemMap), so a resize rehashes only the index entries
// (key, handle and the 4-byte last_seen, which stays with the key) and no
// row moves.  Handles come from a free stack (handles of erased keys) and
// then a bump pointer; an insert pass takes its handles with a count /
// prefix-sum / assign sequence, so no counter is shared by the keys of a
// call.
//
// Probing (this library's layout, not the pages'): the M slots form
// min(16, M)-slot buckets, one 128-byte line of keys each.  A key's walk
// visits bucket b_t = b_0 + t*S mod (M/16) with S odd, so by Theorem 1 over the
// buckets every bucket -- hence every slot -- is on the walk.  Within a bucket
// the slots are taken in order.  A group of G lanes (1, 2, 4, 8 or 16) works
// on one key, each lane holding 16/G consecutive slots of the bucket, so a
// wavefront keeps 64/G keys in flight; the group loads the bucket's 128-byte
// line together and ballots decide found / first free slot / EMPTY seen.  An insert claims the
// first free (EMPTY or TOMBSTONE) slot of the walk with a 64-bit CAS; if the
// CAS loses, the returned key is either the key itself (FOUND) or another
// key, and the walk resumes right after that slot.
#include <cstdlib>

#include "probe.h"
#include "debug.h"
#include "scan.h"

namespace htl {

namespace {
thread_local std::string g_last_error;
constexpr uint64_t kProbeSalt = 0x2545F4914F6CDD1Dull;
// Workgroups of the find-or-insert kernels at most (each loops over its
// share): n_max is only a bound on the keys (the dedup's output
// size), so a full grid would mostly launch blocks that find nothing to do,
// and on a logged table every block also adds its per-step counts.  Per step
// with 2^13 / 2^14 / 2^15: large table 0.594 / 0.597 / 0.597 ms, online
// forward (logged) 0.381 / - / 0.391 ms, merged tables unchanged; 2^12 0.600.
constexpr int64_t kProbeGridMax = 1 << 13;
constexpr int64_t kEraseGridMax = 1 << 11;   // workgroups of the erase kernel at most
}  // namespace

int probe_lanes() {
    static int lanes = [] {
        const char* e = getenv("HTL_PROBE_LANES");
        int v = e ? atoi(e) : 2;
        return (v == 1 || v == 2 || v == 4 || v == 8 || v == 16) ? v : 2;
    }();
    return lanes;
}

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
htl_status fail(htl_status code, const std::string& msg) {
    g_last_error = msg;
    return code;
}
htl_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(HTL_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    return HTL_OK;
}

// --------------------------------------------------------------- kernels --
__global__ void k_fill_i64(int64_t* __restrict__ p, int64_t n, int64_t value) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t value) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// ------------------------------------------------------- access log --
// Thread 0 of block 0 of a logged find-or-insert: the step's record (new
// when the step is), the head for the next call (the other word of the
// pair, which no block of this call reads), and the checks that keep the
// log complete -- the ring must not wrap onto entries at or after the tail,
// and the live steps must lie within kLogSteps of each other, so that a
// step record is only reused once its old step has no live key.
__device__ void log_begin_call(const LogDev& L, int par, uint64_t head0, int64_t n, uint32_t step, int first) {
    LogState* s = L.st;
    if (first) {
        s->s_min = step;
        s->tail = head0;
    }
    LogSeg* g = L.segs + (step & kLogStepMask);
    if (g->step != step) {
        g->step = step;
        g->begin = head0;
    }
    g->end = head0 + (uint64_t)n;
    s->head[par ^ 1] = head0 + (uint64_t)n;
    if ((int64_t)(step - s->s_min) >= kLogSteps || head0 + (uint64_t)n - s->tail > L.cap_mask + 1) s->bad = 1;
}

// Partial count `blockIdx.x mod kLogSubs` of the step.
__device__ __forceinline__ void log_count_add(const LogDev& L, uint32_t step, int64_t delta) {
    const int64_t at = ((int64_t)(step & kLogStepMask) * kLogSubs + (blockIdx.x & (kLogSubs - 1))) * kLogCntStride;
    atomicAdd((unsigned long long*)&L.cnt[at], (unsigned long long)delta);
}

// The LDS bins of a block, added to the step records once: bin b holds keys
// that left step ref - 1 - b (down) or ref + b (up).
__device__ __forceinline__ void log_flush_bins(const LogDev& L, const int* s_bins, uint32_t ref, bool down) {
    for (int b = threadIdx.x; b < kLogBins; b += blockDim.x)
        if (s_bins[b]) log_count_add(L, down ? ref - 1u - (uint32_t)b : ref + (uint32_t)b, -(int64_t)s_bins[b]);
}

// Lane gl == 0 of key i's group in a logged find-or-insert, before the
// stamp: key i's ring entry, and its step counts (new stamps summed in
// s_log[kLogBins], the steps they leave in s_log[step - 1 - old]).  A FOUND
// key already stamped with `step` (an earlier call of the same step) keeps
// its entry.
__device__ __forceinline__ void log_stamp(const LogDev& L, const TableDev& T, int* s_log, uint64_t head0, int64_t i,
                                          int st, int64_t slot, uint32_t step) {
    uint64_t e = kLogNoSlot;
    if (st == HT_FOUND || st == HT_INSERTED) {
        const uint32_t old = st == HT_FOUND ? T.last_seen[slot] : kLsDead;
        if (st == HT_INSERTED || old != step) {
            e = (uint64_t)(uint32_t)slot | ((uint64_t)step << 32);
            atomicAdd(&s_log[kLogBins], 1);
            if (old != kLsDead) {
                const uint32_t d = step - 1u - old;    // old < step: steps of a logged table never decrease
                if (old < step && d < (uint32_t)kLogBins) atomicAdd(&s_log[d], 1);
                else log_count_add(L, old, -1);
            }
        }
    }
    L.entries[(head0 + (uint64_t)i) & L.cap_mask] = e;
}

// Block-level set-up and commit of a logged call's counts.
__device__ __forceinline__ void log_block_init(int* s_log) {
    for (int b = threadIdx.x; b <= kLogBins; b += blockDim.x) s_log[b] = 0;
}
__device__ __forceinline__ void log_block_commit(const LogDev& L, const int* s_log, uint32_t step) {
    log_flush_bins(L, s_log, step, true);
    if (threadIdx.x == 0 && s_log[kLogBins]) log_count_add(L, step, s_log[kLogBins]);
}

// WAVE_ROWS (rows of a multiple of 16 bytes): the whole wave writes the new
// rows of its groups together, after the probes; else each group writes its
// own key's row.  LOG: the table keeps an access log (above).
template <int G, bool WAVE_ROWS, bool LOG>
__global__ __launch_bounds__(kProbeBlock) void k_find_or_insert(
    TableDev T, const int64_t* __restrict__ keys, int64_t n_max, const int64_t* __restrict__ n_dev,
    uint32_t step, int32_t* __restrict__ slots, uint8_t* __restrict__ status, LogDev L, int par, int first) {
    const int64_t n = clamp_count(n_max, n_dev);
    __shared__ int s_log[LOG ? kLogBins + 1 : 1];
    uint64_t head0 = 0;
    if (LOG) {
        log_block_init(s_log);
        head0 = L.st->head[par];
        if (blockIdx.x == 0 && threadIdx.x == 0) log_begin_call(L, par, head0, n, step, first);
        __syncthreads();
    }
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int64_t group0 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / G;
    const int64_t ngroups = (int64_t)gridDim.x * blockDim.x / G;
    // The loop runs the same number of times on every lane of a wave (its
    // bound is the wave's first group), so the whole wave can write rows.
    const int64_t wave0 = group0 - lane / G;

    for (int64_t iw = wave0; iw < n; iw += ngroups) {
        const int64_t i = iw + lane / G;
        int st = HT_NOT_FOUND;
        int64_t slot = -1, k = 0;
        if (i < n) {
            k = keys[i];
            st = find_or_insert_key<G>(T, k, gl, gshift, &slot);
            if (!WAVE_ROWS && st == HT_INSERTED) write_initial_row<G>(T, slot, k, gl);
            if (gl == 0) {
                if (LOG) log_stamp(L, T, s_log, head0, i, st, slot, step);
                if ((st == HT_FOUND || st == HT_INSERTED) && T.last_seen) T.last_seen[slot] = step;
                slots[i] = (int32_t)slot;
                status[i] = (uint8_t)st;
            }
        }
        if (WAVE_ROWS) write_initial_rows_wave<G>(T, st == HT_INSERTED, slot, k);
    }
    if (LOG) {
        __syncthreads();
        log_block_commit(L, s_log, step);
    }
}

// LOG: each erased key takes one from its last_seen step's count (LDS bins
// from s_min up, which is where eviction victims come from).
template <int G, bool LOG>
__global__ __launch_bounds__(kProbeBlock) void k_erase(TableDev T, const int64_t* __restrict__ keys,
                                                       int64_t n, uint8_t* __restrict__ status,
                                                       int32_t* __restrict__ row_tmp, LogDev L) {
    __shared__ int s_log[LOG ? kLogBins : 1];
    uint32_t smin = 0;
    if (LOG) {
        for (int b = threadIdx.x; b < kLogBins; b += blockDim.x) s_log[b] = 0;
        smin = L.st->s_min;
        __syncthreads();
    }
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int W = 1 << T.bucket_log2;
    const uint64_t nb = T.bucket_mask + 1;
    const int64_t group0 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / G;
    const int64_t ngroups = (int64_t)gridDim.x * blockDim.x / G;
    for (int64_t i = group0; i < n; i += ngroups) {
        const int64_t k = keys[i];
        int st = HT_NOT_FOUND;
        if (k != kEmpty && k != kTomb) {
            const uint64_t h = mix64((uint64_t)k ^ T.salt);
            const uint64_t S = ((h >> 32) | 1ull) & T.bucket_mask;
            uint64_t b = h & T.bucket_mask;
            for (uint64_t t = 0; t < nb; ++t) {
                const int64_t base = (int64_t)(b << T.bucket_log2);
                int hit, fs;
                int64_t fv;
                bool has_empty;
                probe_bucket<G>(T.keys + base, k, gl, gshift, 0, W, hit, fs, fv, has_empty);
                if (hit >= 0) {
                    int64_t old = 0;
                    if (gl == 0) old = cas_key(T.keys + base + hit, k, kTomb);
                    old = __shfl(old, gshift);
                    st = (old == k) ? HT_ERASED : HT_NOT_FOUND;
                    if (gl == 0 && st == HT_ERASED && row_tmp) row_tmp[i] = T.rowid[base + hit];
                    if (LOG && gl == 0 && st == HT_ERASED) {
                        const uint32_t old = T.last_seen[base + hit];
                        if (old != kLsDead) {
                            const uint32_t d = old - smin;
                            if (old >= smin && d < (uint32_t)kLogBins) atomicAdd(&s_log[d], 1);
                            else log_count_add(L, old, -1);
                        }
                    }
                    if (gl == 0 && st == HT_ERASED && T.last_seen) T.last_seen[base + hit] = kLsDead;
                    break;
                }
                if (has_empty) break;
                b = (b + S) & T.bucket_mask;
            }
        }
        if (gl == 0 && status) status[i] = (uint8_t)st;
    }
    if (LOG) {
        __syncthreads();
        log_flush_bins(L, s_log, smin, false);
    }
}

// --------------------------------------------------- growable tables --
constexpr int kChunkKeys = 64;    // keys per handle-allocation chunk
constexpr int kAssignLanes = 4;   // lanes per key in the assign pass: 64 keys per 256-thread block

// Pass 1 of an insert into a growable table: probe and claim slots, stamp
// last_seen (kept per slot); the slot goes to slots[i] for pass 3, no row
// is written yet.
template <int G, bool LOG>
__global__ __launch_bounds__(kProbeBlock) void k_foi_claim(TableDev T, const int64_t* __restrict__ keys,
                                                          int64_t n_max, const int64_t* __restrict__ n_dev,
                                                          uint32_t step, int32_t* __restrict__ slots,
                                                          uint8_t* __restrict__ status, LogDev L, int par,
                                                          int first) {
    const int64_t n = clamp_count(n_max, n_dev);
    __shared__ int s_log[LOG ? kLogBins + 1 : 1];
    uint64_t head0 = 0;
    if (LOG) {
        log_block_init(s_log);
        head0 = L.st->head[par];
        if (blockIdx.x == 0 && threadIdx.x == 0) log_begin_call(L, par, head0, n, step, first);
        __syncthreads();
    }
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int64_t group0 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / G;
    const int64_t ngroups = (int64_t)gridDim.x * blockDim.x / G;
    for (int64_t i = group0; i < n; i += ngroups) {
        int64_t slot;
        const int st = find_or_insert_key<G>(T, keys[i], gl, gshift, &slot);
        if (gl == 0) {
            if (LOG) log_stamp(L, T, s_log, head0, i, st, slot, step);
            if ((st == HT_FOUND || st == HT_INSERTED) && T.last_seen) T.last_seen[slot] = step;
            slots[i] = (int32_t)slot;
            status[i] = (uint8_t)st;
        }
    }
    if (LOG) {
        __syncthreads();
        log_block_commit(L, s_log, step);
    }
}

// Per chunk of kChunkKeys keys (one wavefront each): how many of its first
// n keys have status `want`.  Writes every one of the nchunks counts.
__global__ void k_chunk_count(const uint8_t* __restrict__ status, int64_t n_max, const int64_t* __restrict__ n_dev,
                              int want, int32_t* __restrict__ cnt, int64_t nchunks) {
    const int64_t n = clamp_count(n_max, n_dev);
    const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t c = wave; c < nchunks; c += nwaves) {
        const int64_t i = c * kChunkKeys + lane_id();
        const bool f = i < n && status[i] == want;
        const int k = __popcll(__ballot(f));
        if (lane_id() == 0) cnt[c] = k;
    }
}

// The handle for the r-th new row of a call: the top of the free stack
// first, then never-used rows.
__device__ __forceinline__ int32_t take_handle(int64_t r, int64_t bump, int64_t nfree,
                                               const int32_t* __restrict__ free_stack) {
    return r < nfree ? free_stack[nfree - 1 - r] : (int32_t)(bump + (r - nfree));
}

// Pass 3: INSERTED keys take handles in key order (rank within the chunk +
// the chunk's prefix), record them at their slot and get their initial row
// (written by the whole wave when WAVE_ROWS); slots[i] becomes the handle.
template <bool WAVE_ROWS>
__global__ __launch_bounds__(kProbeBlock) void k_foi_assign(TableDev T, const int64_t* __restrict__ keys,
                                                           int64_t n_max, const int64_t* __restrict__ n_dev,
                                                           const int32_t* __restrict__ chunk_off,
                                                           const int64_t* __restrict__ state,
                                                           const int32_t* __restrict__ free_stack,
                                                           int32_t* __restrict__ slots,
                                                           const uint8_t* __restrict__ status) {
    constexpr int G = kAssignLanes;
    __shared__ int s_wave[kProbeBlock / 64];
    const int64_t n = clamp_count(n_max, n_dev);
    const int64_t bump = state[0], nfree = state[1];
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    for (int64_t c = blockIdx.x; c * kChunkKeys < n; c += gridDim.x) {
        const int64_t i = c * kChunkKeys + threadIdx.x / G;
        const int st = i < n ? (int)status[i] : -1;
        const bool ins = st == HT_INSERTED;
        const uint64_t m = __ballot(gl == 0 && ins);
        if (lane == 0) s_wave[wid] = __popcll(m);
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wid; ++w) before += s_wave[w];
        __syncthreads();
        int64_t row = 0, key = 0;
        if (ins) {
            const int64_t slot = slots[i];
            const int64_t r = chunk_off[c] + before + __popcll(m & ((1ull << gshift) - 1ull));
            row = take_handle(r, bump, nfree, free_stack);
            key = keys[i];
            if (!WAVE_ROWS) write_initial_row<G>(T, row, key, gl);
            if (gl == 0) {
                T.rowid[slot] = (int32_t)row;
                slots[i] = (int32_t)row;
            }
        }
        if (WAVE_ROWS) write_initial_rows_wave<G>(T, ins, row, key);
    }
}

// Pass 4: FOUND keys read their slot's handle (after pass 3, so a key that
// another entry of the same call inserted reads the handle just recorded);
// slots[i] becomes the handle.
__global__ void k_foi_found(const TableDev T, int64_t n_max, const int64_t* __restrict__ n_dev,
                            int32_t* __restrict__ slots, const uint8_t* __restrict__ status) {
    const int64_t n = clamp_count(n_max, n_dev);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        if (status[i] == HT_FOUND) slots[i] = T.rowid[slots[i]];
}

// Pass 5 (one thread): the handles taken leave the free stack / bump pointer.
__global__ void k_foi_finish(int64_t* __restrict__ state, const int32_t* __restrict__ total) {
    const int64_t t = *total, nfree = state[1];
    const int64_t take = t < nfree ? t : nfree;
    state[1] = nfree - take;
    state[0] += t - take;
}

// Erase of a growable table: handles of the erased keys go on the free
// stack (rank in key order, after the current top).
__global__ void k_erase_push(const uint8_t* __restrict__ status, const int32_t* __restrict__ row_tmp, int64_t n,
                             const int32_t* __restrict__ chunk_off, const int64_t* __restrict__ state,
                             int32_t* __restrict__ free_stack) {
    const int64_t nfree = state[1];
    const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t c = wave; c * kChunkKeys < n; c += nwaves) {
        const int64_t i = c * kChunkKeys + lane_id();
        const bool f = i < n && status[i] == HT_ERASED;
        const uint64_t m = __ballot(f);
        if (f) free_stack[nfree + chunk_off[c] + __popcll(m & lanemask_lt())] = row_tmp[i];
    }
}

__global__ void k_erase_finish(int64_t* __restrict__ state, const int32_t* __restrict__ total) {
    state[1] += *total;
}

// Resize: each wavefront loads 64 consecutive old slots (one per lane),
// ballots the live ones, and its 64/G groups of G lanes re-insert them,
// with their handle and last_seen, into the new index (keys are distinct,
// so each lands in a free slot; the new index holds no tombstones).
template <int G>
__global__ __launch_bounds__(kProbeBlock) void k_rehash(TableDev O, TableDev N) {
    constexpr int GROUPS = 64 / G;
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int grp = lane / G;
    const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t s0 = wave * 64; s0 < O.capacity; s0 += nwaves * 64) {
        const int64_t s = s0 + lane;
        const int64_t k = s < O.capacity ? O.keys[s] : kEmpty;
        const bool live = k != kEmpty && k != kTomb;
        const int32_t rid = live ? O.rowid[s] : 0;
        const uint32_t ls = (live && O.last_seen) ? O.last_seen[s] : 0u;
        uint64_t mask = __ballot(live);
        while (mask) {
            // group g takes the g-th live lane of what is left
            uint64_t m = mask;
            for (int q = 0; q < grp && m; ++q) m &= m - 1;
            const int src = m ? __builtin_ctzll(m) : -1;
            const int64_t key = __shfl(k, src < 0 ? 0 : src);
            const int32_t r = __shfl(rid, src < 0 ? 0 : src);
            const uint32_t l = __shfl(ls, src < 0 ? 0 : src);
            int64_t ns = -1;
            int st = HT_FULL;
            if (src >= 0) st = find_or_insert_key<G>(N, key, gl, gshift, &ns);
            if (gl == 0 && src >= 0 && st == HT_INSERTED) {
                N.rowid[ns] = r;
                if (N.last_seen) N.last_seen[ns] = l;
            }
            for (int q = 0; q < GROUPS && mask; ++q) mask &= mask - 1;
        }
    }
}

// ------------------------------------------------------- checkpoint --
// Export of a slot range in chunks of kExpChunk slots, one block each: count
// the live slots, prefix the counts, then write each chunk's live entries in
// slot order (MTGR section 5: compact key scanning).  Keys are loaded
// coalesced: slot j * kExpThreads + tid of the chunk belongs to thread tid
// (load round j), so slot order is (round, wave, lane) order and a chunk's
// prefix is taken over its kExpRounds x (kExpThreads / 64) wave counts.
constexpr int kExpChunk = 4096;
constexpr int kExpThreads = 256;
constexpr int kExpRounds = kExpChunk / kExpThreads;
constexpr int kExpWaves = kExpThreads / 64;

__device__ __forceinline__ bool is_live(int64_t k) { return k != kEmpty && k != kTomb; }

__global__ __launch_bounds__(kExpThreads) void k_exp_count(TableDev T, int64_t begin, int64_t end, int64_t nchunks,
                                                          int32_t* __restrict__ cnt) {
    __shared__ int s_wave[kExpWaves];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t s0 = begin + c * kExpChunk + threadIdx.x;
        int mine = 0;
#pragma unroll
        for (int j = 0; j < kExpRounds; ++j) {
            const int64_t s = s0 + (int64_t)j * kExpThreads;
            if (s < end && is_live(T.keys[s])) ++mine;
        }
        for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off);
        if (lane_id() == 0) s_wave[threadIdx.x >> 6] = mine;
        __syncthreads();
        if (threadIdx.x == 0) {
            int tot = 0;
            for (int w = 0; w < kExpWaves; ++w) tot += s_wave[w];
            cnt[c] = tot;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kExpThreads) void k_exp_write(TableDev T, int64_t begin, int64_t end, int64_t nchunks,
                                                          const int32_t* __restrict__ off,
                                                          int64_t* __restrict__ keys_out, void* __restrict__ rows_out,
                                                          uint32_t* __restrict__ ls_out, float* __restrict__ m_out,
                                                          float* __restrict__ v_out, int32_t* __restrict__ slots_out) {
    __shared__ int s_pre[kExpRounds * kExpWaves];   // per (round, wave): live entries before it in the chunk
    __shared__ int s_total;
    __shared__ int32_t s_row[kExpChunk];            // row handle of the chunk's e-th live entry
    __shared__ int32_t s_slot[kExpChunk];           // its slot
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t s0 = begin + c * kExpChunk + threadIdx.x;
        int64_t k[kExpRounds];
#pragma unroll
        for (int j = 0; j < kExpRounds; ++j) {
            const int64_t s = s0 + (int64_t)j * kExpThreads;
            k[j] = s < end ? T.keys[s] : kEmpty;
        }
        uint64_t m[kExpRounds];
#pragma unroll
        for (int j = 0; j < kExpRounds; ++j) {
            m[j] = __ballot(is_live(k[j]));
            if (lane == 0) s_pre[j * kExpWaves + wid] = __popcll(m[j]);
        }
        __syncthreads();
        if (threadIdx.x < 64) {                       // exclusive scan of the 64 counts
            const int v = threadIdx.x < kExpRounds * kExpWaves ? s_pre[threadIdx.x] : 0;
            int incl = v;
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            if (threadIdx.x < kExpRounds * kExpWaves) s_pre[threadIdx.x] = incl - v;
            if (threadIdx.x == 63) s_total = incl;
        }
        __syncthreads();
        const int total = s_total;
        const int64_t base = off[c];
        const uint64_t below = lanemask_lt();
#pragma unroll
        for (int j = 0; j < kExpRounds; ++j) {
            if (m[j] & (1ull << lane)) {
                const int pos = s_pre[j * kExpWaves + wid] + __popcll(m[j] & below);
                const int64_t s = s0 + (int64_t)j * kExpThreads;
                if (keys_out) keys_out[base + pos] = k[j];
                s_slot[pos] = (int32_t)s;
                s_row[pos] = (int32_t)row_of(T, s);
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < total; e += kExpThreads) {
            if (ls_out) ls_out[base + e] = T.last_seen ? T.last_seen[s_slot[e]] : 0u;
            if (slots_out) slots_out[base + e] = s_row[e];
        }
        if (rows_out) {
            if ((row_bytes & 15) == 0) {
                const int vpr = (int)(row_bytes >> 4);
                const u32x4* src = reinterpret_cast<const u32x4*>(T.rows);
                u32x4* dst = reinterpret_cast<u32x4*>(rows_out);
                for (int64_t q = threadIdx.x; q < (int64_t)total * vpr; q += kExpThreads) {
                    const int64_t e = q / vpr, v = q - e * vpr;
                    dst[(base + e) * vpr + v] = src[(int64_t)s_row[e] * vpr + v];
                }
            } else if (T.elem_bytes == 4) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(T.rows);
                uint32_t* dst = reinterpret_cast<uint32_t*>(rows_out);
                for (int64_t q = threadIdx.x; q < (int64_t)total * T.dim; q += kExpThreads) {
                    const int64_t e = q / T.dim, j = q - e * T.dim;
                    dst[(base + e) * T.dim + j] = src[(int64_t)s_row[e] * T.dim + j];
                }
            } else {
                const uint16_t* src = reinterpret_cast<const uint16_t*>(T.rows);
                uint16_t* dst = reinterpret_cast<uint16_t*>(rows_out);
                for (int64_t q = threadIdx.x; q < (int64_t)total * T.dim; q += kExpThreads) {
                    const int64_t e = q / T.dim, j = q - e * T.dim;
                    dst[(base + e) * T.dim + j] = src[(int64_t)s_row[e] * T.dim + j];
                }
            }
        }
        if (m_out || v_out) {
            for (int64_t q = threadIdx.x; q < (int64_t)total * T.dim; q += kExpThreads) {
                const int64_t e = q / T.dim, j = q - e * T.dim;
                const int64_t from = (int64_t)s_row[e] * T.dim + j;
                if (m_out) m_out[(base + e) * T.dim + j] = T.m[from];
                if (v_out) v_out[(base + e) * T.dim + j] = T.v[from];
            }
        }
        __syncthreads();
    }
}

__global__ void k_exp_total(const int32_t* __restrict__ total, int64_t* __restrict__ n_dev) { *n_dev = *total; }

__global__ void k_zero_i64(int64_t* p) { *p = 0; }

// Import: rows and Adam moments of the keys that are live after the
// find-or-insert (FOUND or INSERTED) are written at their handle.
__global__ void k_imp_rows(TableDev T, int64_t n, const int32_t* __restrict__ handles,
                           const uint8_t* __restrict__ status, const void* __restrict__ rows_in,
                           const float* __restrict__ m_in, const float* __restrict__ v_in) {
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if ((row_bytes & 15) == 0) {
        const int vpr = (int)(row_bytes >> 4);
        const u32x4* src = reinterpret_cast<const u32x4*>(rows_in);
        u32x4* dst = reinterpret_cast<u32x4*>(T.rows);
        for (int64_t q = t0; q < n * vpr; q += stride) {
            const int64_t i = q / vpr, v = q - i * vpr;
            const int st = status[i];
            if (st == HT_FOUND || st == HT_INSERTED) dst[(int64_t)handles[i] * vpr + v] = src[i * vpr + v];
        }
    } else {
        for (int64_t q = t0; q < n * T.dim; q += stride) {
            const int64_t i = q / T.dim, j = q - i * T.dim;
            const int st = status[i];
            if (st != HT_FOUND && st != HT_INSERTED) continue;
            const int64_t to = (int64_t)handles[i] * T.dim + j;
            if (T.elem_bytes == 4)
                reinterpret_cast<uint32_t*>(T.rows)[to] = reinterpret_cast<const uint32_t*>(rows_in)[i * T.dim + j];
            else
                reinterpret_cast<uint16_t*>(T.rows)[to] = reinterpret_cast<const uint16_t*>(rows_in)[i * T.dim + j];
        }
    }
    if (m_in) {
        for (int64_t q = t0; q < n * T.dim; q += stride) {
            const int64_t i = q / T.dim, j = q - i * T.dim;
            const int st = status[i];
            if (st != HT_FOUND && st != HT_INSERTED) continue;
            const int64_t to = (int64_t)handles[i] * T.dim + j;
            T.m[to] = m_in[i * T.dim + j];
            T.v[to] = v_in[i * T.dim + j];
        }
    }
}

// Import: last_seen of the live keys, at their slot (found again by a walk:
// in a growable table the handle is not the slot).
template <int G>
__global__ __launch_bounds__(kProbeBlock) void k_imp_ls(TableDev T, const int64_t* __restrict__ keys, int64_t n,
                                                       const uint8_t* __restrict__ status,
                                                       const uint32_t* __restrict__ ls_in) {
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int64_t group0 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / G;
    const int64_t ngroups = (int64_t)gridDim.x * blockDim.x / G;
    for (int64_t i = group0; i < n; i += ngroups) {
        const int st = status[i];
        if (st != HT_FOUND && st != HT_INSERTED) continue;
        const int64_t slot = find_key<G>(T, keys[i], gl, gshift);
        // kLsDead marks dead slots: an imported stamp takes at most the step below it
        if (gl == 0 && slot >= 0) T.last_seen[slot] = ls_in[i] < kLsDead ? ls_in[i] : kLsDead - 1u;
    }
}

// ------------------------------------------------------------ host side --
// Every slot EMPTY; where last_seen is kept, every slot's last_seen dead.
htl_status fill_keys_empty(const TableDev& T, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_i64, dim3(grid_for(T.capacity, 256 * 8, 1 << 16)), dim3(256), 0, s,
                       T.keys, T.capacity, kEmpty);
    if (T.last_seen)
        hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(T.capacity, 256 * 8, 1 << 16)), dim3(256), 0, s,
                           T.last_seen, T.capacity, kLsDead);
    return check_launch("clear table keys");
}

// Access log: every step record empty, every count zero, the ring empty.
__global__ void k_log_reset(LogSeg* __restrict__ segs, int64_t* __restrict__ cnt, LogState* __restrict__ st) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < kLogSteps; i += (int64_t)gridDim.x * blockDim.x) {
        segs[i].step = 0xFFFFFFFFu;
        segs[i].pad = 0u;
        segs[i].begin = 0;
        segs[i].end = 0;
    }
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < kLogSteps * kLogSubs;
         i += (int64_t)gridDim.x * blockDim.x)
        cnt[i * kLogCntStride] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->head[0] = st->head[1] = 0;
        st->tail = 0;
        st->s_min = 0u;
        st->bad = 0;
    }
}

__global__ void k_log_state(const LogState* __restrict__ st, int par, int host_ok, int64_t* __restrict__ out) {
    out[0] = (host_ok && !st->bad) ? 1 : 0;
    out[1] = (int64_t)st->head[par];
    out[2] = (int64_t)st->tail;
    out[3] = (int64_t)st->s_min;
}

// Rebuild of an access log from the table itself: [0] min and [1] max
// last_seen over the live slots, [2] their count (one atomic of each per
// block, over a persistent grid).
__global__ void k_log_range(const uint32_t* __restrict__ ls, int64_t M, unsigned long long* __restrict__ out) {
    __shared__ uint32_t s_lo, s_hi;
    __shared__ unsigned long long s_n;
    if (threadIdx.x == 0) {
        s_lo = 0xFFFFFFFFu;
        s_hi = 0u;
        s_n = 0ull;
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    unsigned long long n = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < M; i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t v = ls[i];
        if (v == kLsDead) continue;
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
        ++n;
    }
    atomicMin(&s_lo, lo);
    atomicMax(&s_hi, hi);
    atomicAdd(&s_n, n);
    __syncthreads();
    if (threadIdx.x == 0) {
        atomicMin(reinterpret_cast<unsigned int*>(out), s_lo);
        atomicMax(reinterpret_cast<unsigned int*>(out + 1), s_hi);
        atomicAdd(out + 2, s_n);
    }
}

// Pass 1 (cursor == nullptr): live slots per step (step - lo < kLogSteps),
// summed in LDS per block and added to cnt.  Pass 2: each block reserves a
// run per step with one add to the step's cursor, then writes its slots'
// entries (slot | step << 32) into the runs.
__global__ __launch_bounds__(256) void k_log_fill(const uint32_t* __restrict__ ls, int64_t M, uint32_t lo,
                                                  uint32_t* __restrict__ cnt, unsigned long long* __restrict__ cursor,
                                                  uint64_t* __restrict__ entries, uint64_t cap_mask) {
    __shared__ uint32_t s_c[kLogSteps];
    __shared__ unsigned long long s_at[kLogSteps];
    for (int b = threadIdx.x; b < kLogSteps; b += blockDim.x) s_c[b] = 0u;
    __syncthreads();
    const int64_t per = (M + gridDim.x - 1) / gridDim.x;       // each block a contiguous range of slots
    const int64_t a = blockIdx.x * per, e = a + per < M ? a + per : M;
    for (int64_t i = a + threadIdx.x; i < e; i += blockDim.x) {
        const uint32_t v = ls[i];
        if (v != kLsDead) atomicAdd(&s_c[v - lo], 1u);
    }
    __syncthreads();
    if (!cursor) {
        for (int b = threadIdx.x; b < kLogSteps; b += blockDim.x)
            if (s_c[b]) atomicAdd(&cnt[b], s_c[b]);
        return;
    }
    for (int b = threadIdx.x; b < kLogSteps; b += blockDim.x)
        s_at[b] = s_c[b] ? atomicAdd(&cursor[b], (unsigned long long)s_c[b]) : 0ull;
    __syncthreads();
    for (int64_t i = a + threadIdx.x; i < e; i += blockDim.x) {
        const uint32_t v = ls[i];
        if (v == kLsDead) continue;
        const unsigned long long at = atomicAdd(&s_at[v - lo], 1ull);
        entries[at & cap_mask] = (uint64_t)(uint32_t)i | ((uint64_t)v << 32);
    }
}

// The rebuilt log's step counts (partial count 0 of each step) and state.
__global__ void k_log_set(int64_t* __restrict__ cntp, const uint32_t* __restrict__ cnt, uint32_t lo, int64_t span,
                          LogState* __restrict__ st, int par, uint64_t head, uint32_t s_min) {
    for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < span; b += (int64_t)gridDim.x * blockDim.x)
        cntp[(int64_t)((lo + (uint32_t)b) & kLogStepMask) * kLogSubs * kLogCntStride] = cnt[b];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->head[par] = head;
        st->tail = 0;
        st->s_min = s_min;
        st->bad = 0;
    }
}

// Ring entries of a table's access log: a quarter of the slots, at least 4096.
int64_t log_capacity(int capacity_log2) {
    return (int64_t)1 << (capacity_log2 - 2 > 12 ? capacity_log2 - 2 : 12);
}

htl_status log_reset(htl_table* t, hipStream_t stream) {
    if (!t->log.entries) return HTL_OK;
    hipLaunchKernelGGL(k_log_reset, dim3(grid_for(kLogSteps * kLogSubs, 256, 256)), dim3(256), 0, stream, t->log.segs,
                       t->log.cnt, t->log.st);
    t->log_ok = true;
    t->log_first = true;
    t->log_par = 0;
    t->erase_pending = false;
    return check_launch("access log reset");
}

htl_status log_alloc(htl_table* t, hipStream_t stream) {
    const int64_t cap = log_capacity(t->capacity_log2);
    if (hipMalloc((void**)&t->log.entries, (size_t)cap * 8) != hipSuccess ||
        hipMalloc((void**)&t->log.segs, (size_t)kLogSteps * sizeof(LogSeg)) != hipSuccess ||
        hipMalloc((void**)&t->log.cnt, (size_t)kLogSteps * kLogSubs * kLogCntStride * 8) != hipSuccess ||
        hipMalloc((void**)&t->log.st, sizeof(LogState)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(HTL_ERR_NOMEM, "ht_create: access log allocation failed");
    }
    t->log.cap_mask = (uint64_t)cap - 1u;
    return log_reset(t, stream);
}

void log_free(htl_table* t) {
    if (t->log.entries) (void)hipFree(t->log.entries);
    if (t->log.segs) (void)hipFree(t->log.segs);
    if (t->log.cnt) (void)hipFree(t->log.cnt);
    if (t->log.st) (void)hipFree(t->log.st);
    t->log = LogDev{};
}

// Whether a find-or-insert at `step` is logged.  Turns the log off (until
// ht_clear) when the call would break its premises: steps never decrease
// along the ring, and no key is inserted at a step that an erase already
// saw (a slot freed and claimed again within one step would give two
// current entries).  Called before max_step is raised.
bool log_foi(htl_table* t, uint32_t step) {
    if (!t->log.entries || !t->log_ok) return false;
    if (!t->log_first && step < t->max_step) {
        t->log_ok = false;
        return false;
    }
    if (t->erase_pending) {
        if (step <= t->erase_step) {
            t->log_ok = false;
            return false;
        }
        t->erase_pending = false;
    }
    return true;
}

hipMemAllocationProp vm_prop(int device) {
    hipMemAllocationProp prop = {};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = device;
    return prop;
}

size_t vm_granularity(int device) {
    const hipMemAllocationProp prop = vm_prop(device);
    size_t g = 0;
    if (hipMemGetAllocationGranularity(&g, &prop, hipMemAllocationGranularityMinimum) != hipSuccess || g == 0)
        g = (size_t)2 << 20;
    return g;
}

htl_status vm_reserve(VmArray& a, size_t bytes, int device) {
    const size_t g = vm_granularity(device);
    a.reserved = align_up(bytes, g);
    if (hipMemAddressReserve(&a.base, a.reserved, 0, nullptr, 0) != hipSuccess) {
        (void)hipGetLastError();
        a.base = nullptr;
        a.reserved = 0;
        return fail(HTL_ERR_DEVICE, "growable table: cannot reserve device address space");
    }
    return HTL_OK;
}

// Maps physical memory so that the first `bytes` of the range are usable.
htl_status vm_map_to(VmArray& a, size_t bytes, int device) {
    const size_t g = vm_granularity(device);
    const size_t need = align_up(bytes, g);
    if (need <= a.mapped) return HTL_OK;
    if (need > a.reserved) return fail(HTL_ERR_INVALID, "growable table: beyond the reserved row space");
    const size_t size = need - a.mapped;
    const hipMemAllocationProp prop = vm_prop(device);
    hipMemGenericAllocationHandle_t h;
    if (hipMemCreate(&h, size, &prop, 0) != hipSuccess) {
        (void)hipGetLastError();
        return fail(HTL_ERR_NOMEM, "growable table: hipMemCreate failed");
    }
    char* at = (char*)a.base + a.mapped;
    if (hipMemMap(at, size, 0, h, 0) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipMemRelease(h);
        return fail(HTL_ERR_DEVICE, "growable table: hipMemMap failed");
    }
    // Access is set over the whole mapped range from the base: on this
    // runtime, setting it on the new chunk alone is refused ("invalid
    // argument") for many chunk sequences, while the whole range never was
    // in repeated trials on MI355X.
    hipMemAccessDesc d = {};
    d.location = prop.location;
    d.flags = hipMemAccessFlagsProtReadWrite;
    if (hipMemSetAccess(a.base, need, &d, 1) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipMemUnmap(at, size);
        (void)hipMemRelease(h);
        return fail(HTL_ERR_DEVICE, "growable table: hipMemSetAccess failed");
    }
    a.handles.push_back(h);
    a.sizes.push_back(size);
    a.mapped = need;
    return HTL_OK;
}

void vm_free(VmArray& a) {
    size_t off = 0;
    for (size_t i = 0; i < a.handles.size(); ++i) {
        (void)hipMemUnmap((char*)a.base + off, a.sizes[i]);
        (void)hipMemRelease(a.handles[i]);
        off += a.sizes[i];
    }
    if (a.base) (void)hipMemAddressFree(a.base, a.reserved);
    a = VmArray{};
}

// Maps the row space of a growable table for `rows` handles.
htl_status grow_row_space(htl_table* t, int64_t rows) {
    TableDev& T = t->dev;
    const size_t rb = (size_t)t->dim * T.elem_bytes;
    htl_status st = vm_map_to(t->vm_rows, (size_t)rows * rb, t->device);
    if (st == HTL_OK && T.m) st = vm_map_to(t->vm_m, (size_t)rows * t->dim * 4, t->device);
    if (st == HTL_OK && T.v) st = vm_map_to(t->vm_v, (size_t)rows * t->dim * 4, t->device);
    return st;
}

// Per-call temporaries of a growable table for up to n keys.
htl_status ensure_tmp(htl_table* t, int64_t n) {
    RowAlloc& A = t->alloc;
    if (n <= A.tmp_keys) return HTL_OK;
    if (A.tmp_base) {
        HTL_HIP(hipDeviceSynchronize());
        (void)hipFree(A.tmp_base);
        A.tmp_base = nullptr;
        A.tmp_keys = 0;
    }
    const int64_t nchunks = ceil_div(n, kChunkKeys);
    size_t off = 0;
    auto take = [&](size_t b) {
        const size_t o = off;
        off = align_up(off + b, 256);
        return o;
    };
    const size_t o_cnt = take((size_t)nchunks * 4), o_off = take((size_t)(nchunks + 1) * 4);
    const size_t o_row = take((size_t)n * 4), o_st = take((size_t)n), o_scan = take(scan_temp_bytes(nchunks));
    if (hipMalloc(&A.tmp_base, off) != hipSuccess) {
        (void)hipGetLastError();
        A.tmp_base = nullptr;
        return fail(HTL_ERR_NOMEM, "growable table: temporaries allocation failed");
    }
    char* b = (char*)A.tmp_base;
    A.chunk_cnt = (int32_t*)(b + o_cnt);
    A.chunk_off = (int32_t*)(b + o_off);
    A.row_tmp = (int32_t*)(b + o_row);
    A.status_tmp = (uint8_t*)(b + o_st);
    A.scan_tmp = b + o_scan;
    A.tmp_keys = n;
    return HTL_OK;
}

void free_temporaries(htl_table* t) {
    RowAlloc& A = t->alloc;
    if (A.tmp_base) (void)hipFree(A.tmp_base);
    if (A.exp_base) (void)hipFree(A.exp_base);
    A.tmp_base = A.exp_base = nullptr;
    A.tmp_keys = A.exp_chunks = 0;
}

void free_growable(htl_table* t) {
    vm_free(t->vm_rows);
    vm_free(t->vm_m);
    vm_free(t->vm_v);
    free_temporaries(t);
    RowAlloc& A = t->alloc;
    if (A.state) (void)hipFree(A.state);
    if (A.free_stack) (void)hipFree(A.free_stack);
    A = RowAlloc{};
    if (t->dev.rowid) (void)hipFree(t->dev.rowid);
    t->dev.rowid = nullptr;
}

// Export temporaries for ranges of up to nchunks chunks.
htl_status ensure_exp(htl_table* t, int64_t nchunks) {
    RowAlloc& A = t->alloc;
    if (nchunks <= A.exp_chunks) return HTL_OK;
    if (A.exp_base) {
        HTL_HIP(hipDeviceSynchronize());
        (void)hipFree(A.exp_base);
        A.exp_base = nullptr;
        A.exp_chunks = 0;
    }
    size_t off = 0;
    auto take = [&](size_t b) {
        const size_t o = off;
        off = align_up(off + b, 256);
        return o;
    };
    const size_t o_cnt = take((size_t)nchunks * 4), o_off = take((size_t)(nchunks + 1) * 4);
    const size_t o_scan = take(scan_temp_bytes(nchunks));
    if (hipMalloc(&A.exp_base, off) != hipSuccess) {
        (void)hipGetLastError();
        A.exp_base = nullptr;
        return fail(HTL_ERR_NOMEM, "ht_export: temporaries allocation failed");
    }
    char* b = (char*)A.exp_base;
    A.exp_cnt = (int32_t*)(b + o_cnt);
    A.exp_off = (int32_t*)(b + o_off);
    A.exp_scan = b + o_scan;
    A.exp_chunks = nchunks;
    return HTL_OK;
}

}  // namespace htl

using namespace htl;

extern "C" {

const char* htl_last_error(void) { return g_last_error.c_str(); }

htl_status ht_create(htl_table** out, int capacity_log2, int dim, htl_dtype dtype,
                     uint64_t init_seed, uint32_t flags, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(out != nullptr, "ht_create: null output handle");
    *out = nullptr;
    HTL_REQUIRE(capacity_log2 >= 1 && capacity_log2 <= HT_MAX_CAPACITY_LOG2,
                "ht_create: capacity_log2 must be in [1, 31]");
    HTL_REQUIRE(dim >= 1 && dim <= 65536, "ht_create: dim must be in [1, 65536]");
    HTL_REQUIRE(dtype == HTL_F32 || dtype == HTL_BF16, "ht_create: dtype must be HTL_F32 or HTL_BF16");
    HTL_REQUIRE((flags & ~(uint32_t)(HT_META_LAST_SEEN | HT_ADAM_STATE | HT_GROWABLE | HT_META_ACCESS_LOG)) == 0,
                "ht_create: unknown flag");
    HTL_REQUIRE(!(flags & HT_META_ACCESS_LOG) || ((flags & HT_META_LAST_SEEN) && capacity_log2 <= 30),
                "ht_create: an access log needs HT_META_LAST_SEEN and capacity_log2 <= 30");
    HTL_REQUIRE(!(flags & HT_ADAM_STATE) || dtype == HTL_F32, "ht_create: Adam state needs an fp32 table");
    const bool growable = (flags & HT_GROWABLE) != 0;
    HTL_REQUIRE(!growable || capacity_log2 <= 30, "ht_create: a growable table needs capacity_log2 <= 30");

    htl_table* t = new htl_table();
    t->capacity_log2 = capacity_log2;
    t->dim = dim;
    t->dtype = dtype;
    t->init_seed = init_seed;
    t->flags = flags;
    t->max_capacity_log2 = growable ? (capacity_log2 + 8 < 30 ? capacity_log2 + 8 : 30) : capacity_log2;
    HTL_HIP(hipGetDevice(&t->device));
    TableDev& T = t->dev;
    T = TableDev{};
    T.capacity = (int64_t)1 << capacity_log2;
    T.bucket_log2 = capacity_log2 < kBucketLog2 ? capacity_log2 : kBucketLog2;
    T.bucket_mask = (uint64_t)(T.capacity >> T.bucket_log2) - 1;
    T.dim = dim;
    T.elem_bytes = dtype == HTL_F32 ? 4 : 2;
    T.dtype = dtype;
    T.init_base = mix64(init_seed);
    T.salt = kProbeSalt;

    auto cleanup = [&]() {
        log_free(t);
        if (T.keys) (void)hipFree(T.keys);
        if (T.last_seen && growable) (void)hipFree(T.last_seen);
        if (growable) {
            free_growable(t);
        } else {
            if (T.rows) (void)hipFree(T.rows);
            if (T.last_seen) (void)hipFree(T.last_seen);
            if (T.m) (void)hipFree(T.m);
            if (T.v) (void)hipFree(T.v);
        }
        delete t;
    };
    const size_t M = (size_t)T.capacity;
    const size_t row_bytes = M * (size_t)dim * (size_t)T.elem_bytes;
    if (growable) {
        int vmm = 0;
        if (hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, t->device) !=
                hipSuccess ||
            !vmm) {
            (void)hipGetLastError();
            cleanup();
            return fail(HTL_ERR_DEVICE, "ht_create: the device does not support virtual memory management");
        }
        const size_t R = (size_t)1 << t->max_capacity_log2;
        htl_status st = vm_reserve(t->vm_rows, R * (size_t)dim * T.elem_bytes, t->device);
        if (st == HTL_OK && (flags & HT_ADAM_STATE)) st = vm_reserve(t->vm_m, R * dim * 4, t->device);
        if (st == HTL_OK && (flags & HT_ADAM_STATE)) st = vm_reserve(t->vm_v, R * dim * 4, t->device);
        if (st == HTL_OK) {
            T.rows = t->vm_rows.base;
            T.m = (float*)t->vm_m.base;
            T.v = (float*)t->vm_v.base;
            st = grow_row_space(t, (int64_t)M);
        }
        if (st == HTL_OK && (hipMalloc((void**)&T.keys, M * sizeof(int64_t)) != hipSuccess ||
                             hipMalloc((void**)&T.rowid, M * 4) != hipSuccess ||
                             ((flags & HT_META_LAST_SEEN) &&
                              hipMalloc((void**)&T.last_seen, M * 4) != hipSuccess) ||
                             hipMalloc((void**)&t->alloc.free_stack, M * 4) != hipSuccess ||
                             hipMalloc((void**)&t->alloc.state, 2 * sizeof(int64_t)) != hipSuccess)) {
            (void)hipGetLastError();
            st = fail(HTL_ERR_NOMEM, "ht_create: device allocation failed");
        }
        if (st == HTL_OK) {
            hipLaunchKernelGGL(k_fill_i64, dim3(1), dim3(64), 0, stream, t->alloc.state, (int64_t)2, (int64_t)0);
            st = check_launch("ht_create: row allocator");
        }
        if (st == HTL_OK) st = fill_keys_empty(T, stream);
        if (st == HTL_OK && (flags & HT_META_ACCESS_LOG)) st = log_alloc(t, stream);
        if (st != HTL_OK) {
            std::string msg = g_last_error;
            cleanup();
            return fail(st, msg);
        }
        *out = t;
        return HTL_OK;
    }
    if (hipMalloc((void**)&T.keys, M * sizeof(int64_t)) != hipSuccess ||
        hipMalloc(&T.rows, row_bytes) != hipSuccess ||
        ((flags & HT_META_LAST_SEEN) && hipMalloc((void**)&T.last_seen, M * 4) != hipSuccess) ||
        ((flags & HT_ADAM_STATE) && (hipMalloc((void**)&T.m, M * dim * 4) != hipSuccess ||
                                     hipMalloc((void**)&T.v, M * dim * 4) != hipSuccess))) {
        (void)hipGetLastError();
        cleanup();
        return fail(HTL_ERR_NOMEM, "ht_create: device allocation failed");
    }
    htl_status st = fill_keys_empty(T, stream);
    if (st == HTL_OK && (flags & HT_META_ACCESS_LOG)) st = log_alloc(t, stream);
    if (st != HTL_OK) {
        std::string msg = g_last_error;
        cleanup();
        return fail(st, msg);
    }
    *out = t;
    return HTL_OK;
}

htl_status ht_destroy(htl_table* t) {
    clear_error();
    if (!t) return HTL_OK;
    int cur = 0;
    HTL_HIP(hipGetDevice(&cur));
    HTL_HIP(hipSetDevice(t->device));
    HTL_HIP(hipDeviceSynchronize());
    TableDev& T = t->dev;
    log_free(t);
    (void)hipFree(T.keys);
    if (t->flags & HT_GROWABLE) {
        if (T.last_seen) (void)hipFree(T.last_seen);
        free_growable(t);
    } else {
        free_temporaries(t);
        (void)hipFree(T.rows);
        if (T.last_seen) (void)hipFree(T.last_seen);
        if (T.m) (void)hipFree(T.m);
        if (T.v) (void)hipFree(T.v);
    }
    delete t;
    HTL_HIP(hipSetDevice(cur));
    return HTL_OK;
}

htl_status ht_clear(htl_table* t, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_clear: null table");
    t->max_step = 0u;
    if (t->flags & HT_GROWABLE) {
        hipLaunchKernelGGL(k_fill_i64, dim3(1), dim3(64), 0, stream, t->alloc.state, (int64_t)2, (int64_t)0);
        htl_status st = check_launch("ht_clear: row allocator");
        if (st != HTL_OK) return st;
    }
    htl_status st = log_reset(t, stream);
    if (st != HTL_OK) return st;
    return fill_keys_empty(t->dev, stream);
}

htl_status ht_resize(htl_table* t, int new_capacity_log2, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_resize: null table");
    HTL_REQUIRE(t->flags & HT_GROWABLE, "ht_resize: the table was not created with HT_GROWABLE");
    t->log_ok = false;   // the rehash moves keys to other slots: logged slots go stale
    HTL_REQUIRE(new_capacity_log2 >= t->capacity_log2 && new_capacity_log2 <= t->max_capacity_log2,
                "ht_resize: new_capacity_log2 must be in [current, created + 8] and <= 30");
    TableDev& O = t->dev;
    TableDev N = O;
    N.capacity = (int64_t)1 << new_capacity_log2;
    N.bucket_log2 = new_capacity_log2 < kBucketLog2 ? new_capacity_log2 : kBucketLog2;
    N.bucket_mask = (uint64_t)(N.capacity >> N.bucket_log2) - 1;
    N.keys = nullptr;
    N.rowid = nullptr;
    N.last_seen = nullptr;
    int32_t* new_stack = nullptr;
    const size_t M2 = (size_t)N.capacity;
    htl_status st = grow_row_space(t, N.capacity);
    if (st != HTL_OK) return st;
    if (hipMalloc((void**)&N.keys, M2 * sizeof(int64_t)) != hipSuccess ||
        hipMalloc((void**)&N.rowid, M2 * 4) != hipSuccess || hipMalloc((void**)&new_stack, M2 * 4) != hipSuccess ||
        (O.last_seen && hipMalloc((void**)&N.last_seen, M2 * 4) != hipSuccess)) {
        (void)hipGetLastError();
        if (N.keys) (void)hipFree(N.keys);
        if (N.rowid) (void)hipFree(N.rowid);
        if (N.last_seen) (void)hipFree(N.last_seen);
        if (new_stack) (void)hipFree(new_stack);
        return fail(HTL_ERR_NOMEM, "ht_resize: device allocation failed");
    }
    st = fill_keys_empty(N, stream);
    if (st == HTL_OK && hipMemcpyAsync(new_stack, t->alloc.free_stack, (size_t)O.capacity * 4,
                                       hipMemcpyDeviceToDevice, stream) != hipSuccess) {
        (void)hipGetLastError();
        st = fail(HTL_ERR_DEVICE, "ht_resize: copy of the free handles failed");
    }
    if (st == HTL_OK) {
        hipLaunchKernelGGL(k_rehash<4>, dim3(grid_for(O.capacity, kProbeBlock, 1 << 16)), dim3(kProbeBlock), 0,
                           stream, O, N);
        st = check_launch("ht_resize: rehash");
    }
    if (st == HTL_OK && hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        st = fail(HTL_ERR_DEVICE, "ht_resize: stream synchronisation failed");
    }
    if (st != HTL_OK) {
        std::string msg = g_last_error;
        (void)hipStreamSynchronize(stream);
        (void)hipFree(N.keys);
        (void)hipFree(N.rowid);
        if (N.last_seen) (void)hipFree(N.last_seen);
        (void)hipFree(new_stack);
        return fail(st, msg);
    }
    (void)hipFree(O.keys);
    (void)hipFree(O.rowid);
    if (O.last_seen) (void)hipFree(O.last_seen);
    (void)hipFree(t->alloc.free_stack);
    t->alloc.free_stack = new_stack;
    t->dev = N;
    t->capacity_log2 = new_capacity_log2;
    return HTL_OK;
}

htl_status ht_find_or_insert(htl_table* t, const int64_t* keys, int64_t n_max, const int64_t* n_dev,
                             uint32_t step, int32_t* slots, uint8_t* status, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_find_or_insert: null table");
    HTL_REQUIRE(n_max >= 0 && n_max < ((int64_t)1 << 31), "ht_find_or_insert: n_max out of range");
    HTL_REQUIRE(!t->dev.last_seen || step != kLsDead,
                "ht_find_or_insert: step 0xFFFFFFFF is reserved on a table that keeps last_seen");
    if (n_max == 0) return HTL_OK;
    HTL_REQUIRE(keys && slots && status, "ht_find_or_insert: null keys/slots/status");
    HTL_REQUIRE(aligned(keys, 8) && aligned(slots, 4) && (!n_dev || aligned(n_dev, 8)),
                "ht_find_or_insert: misaligned pointer");
    const bool logged = log_foi(t, step);
    if (step > t->max_step) t->max_step = step;
    const int par = t->log_par, first = t->log_first ? 1 : 0;
    // a logged launch wrote the other head word: the next call reads it
    auto logged_launch = [&]() {
        if (logged) {
            t->log_par ^= 1;
            t->log_first = false;
        }
    };
    const int G = probe_lanes();
    // n_max is an upper bound (the dedup output's size: N, with U < N keys
    // real); a persistent grid keeps the blocks past U from costing launches.
    const unsigned grid = grid_for(n_max, kProbeBlock / G, kProbeGridMax);
    if (t->flags & HT_GROWABLE) {
        // claim slots, count the inserts per chunk, prefix them, hand out rows
        htl_status st = ensure_tmp(t, n_max);
        if (st != HTL_OK) return st;
        RowAlloc& A = t->alloc;
        const int64_t nchunks = ceil_div(n_max, kChunkKeys);
#define HTL_CLAIM(GG)                                                                                          \
    if (logged)                                                                                                \
        hipLaunchKernelGGL((k_foi_claim<GG, true>), dim3(grid), dim3(kProbeBlock), 0, stream, t->dev, keys,    \
                           n_max, n_dev, step, slots, status, t->log, par, first);                            \
    else                                                                                                       \
        hipLaunchKernelGGL((k_foi_claim<GG, false>), dim3(grid), dim3(kProbeBlock), 0, stream, t->dev, keys,   \
                           n_max, n_dev, step, slots, status, t->log, par, first)
        switch (G) {
            case 1: HTL_CLAIM(1); break;
            case 2: HTL_CLAIM(2); break;
            case 8: HTL_CLAIM(8); break;
            case 16: HTL_CLAIM(16); break;
            default: HTL_CLAIM(4); break;
        }
#undef HTL_CLAIM
        logged_launch();
        hipLaunchKernelGGL(k_chunk_count, dim3(grid_for(nchunks, 4, 1 << 16)), dim3(256), 0, stream, status, n_max,
                           n_dev, (int)HT_INSERTED, A.chunk_cnt, nchunks);
        st = scan_exclusive_i32(A.chunk_cnt, A.chunk_off, nchunks, nullptr, kScanIdentity, 1, A.scan_tmp, stream);
        if (st != HTL_OK) return st;
        if (((t->dev.dim * t->dev.elem_bytes) & 15) == 0)
            hipLaunchKernelGGL(k_foi_assign<true>, dim3(grid_for(nchunks, 1, 1 << 14)), dim3(kProbeBlock), 0, stream,
                               t->dev, keys, n_max, n_dev, A.chunk_off, A.state, A.free_stack, slots, status);
        else
            hipLaunchKernelGGL(k_foi_assign<false>, dim3(grid_for(nchunks, 1, 1 << 14)), dim3(kProbeBlock), 0, stream,
                               t->dev, keys, n_max, n_dev, A.chunk_off, A.state, A.free_stack, slots, status);
        hipLaunchKernelGGL(k_foi_found, dim3(grid_for(n_max, 256 * 4)), dim3(256), 0, stream, t->dev, n_max, n_dev,
                           slots, status);
        hipLaunchKernelGGL(k_foi_finish, dim3(1), dim3(1), 0, stream, A.state, A.chunk_off + nchunks);
        debug_check_foi(t->dev, keys, n_max, n_dev, slots, status, stream);
        debug_check_log(t, stream);
        return check_launch("ht_find_or_insert");
    }
#define HTL_FOI_L(GG, WR, LG)                                                                             \
    hipLaunchKernelGGL((k_find_or_insert<GG, WR, LG>), dim3(grid), dim3(kProbeBlock), 0, stream, t->dev, \
                       keys, n_max, n_dev, step, slots, status, t->log, par, first)
#define HTL_FOI(GG)                  \
    if (logged) {                    \
        if (wave_rows)               \
            HTL_FOI_L(GG, true, true);  \
        else                         \
            HTL_FOI_L(GG, false, true); \
    } else if (wave_rows)            \
        HTL_FOI_L(GG, true, false);     \
    else                             \
        HTL_FOI_L(GG, false, false)
    const bool wave_rows = ((t->dev.dim * t->dev.elem_bytes) & 15) == 0;
    switch (G) {
        case 1: HTL_FOI(1); break;
        case 2: HTL_FOI(2); break;
        case 8: HTL_FOI(8); break;
        case 16: HTL_FOI(16); break;
        default: HTL_FOI(4); break;
    }
#undef HTL_FOI
#undef HTL_FOI_L
    logged_launch();
    debug_check_foi(t->dev, keys, n_max, n_dev, slots, status, stream);
    debug_check_log(t, stream);
    return check_launch("ht_find_or_insert");
}

htl_status ht_erase(htl_table* t, const int64_t* keys, int64_t n, uint8_t* status, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_erase: null table");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "ht_erase: n out of range");
    if (n == 0) return HTL_OK;
    HTL_REQUIRE(keys && aligned(keys, 8), "ht_erase: null or misaligned keys");
    const bool logged = t->log.entries && t->log_ok;
    if (logged && !t->log_first) {
        t->erase_pending = true;
        t->erase_step = t->max_step;
    }
    // at most 2^11 workgroups, each looping: fewer blocks flush their LDS step
    // counts (online erase of 5% of the live keys: 28.7 -> 27.6 us; 2^12 28.0)
    const unsigned egrid = grid_for(n, kProbeBlock / 8, kEraseGridMax);
    auto erase = [&](uint8_t* stat, int32_t* row_tmp) {
        if (logged)
            hipLaunchKernelGGL((k_erase<8, true>), dim3(egrid), dim3(kProbeBlock), 0, stream, t->dev, keys, n, stat,
                               row_tmp, t->log);
        else
            hipLaunchKernelGGL((k_erase<8, false>), dim3(egrid), dim3(kProbeBlock), 0, stream, t->dev, keys, n, stat,
                               row_tmp, t->log);
    };
    if (t->flags & HT_GROWABLE) {
        // erased keys' row handles go back on the free stack, in key order
        htl_status st = ensure_tmp(t, n);
        if (st != HTL_OK) return st;
        RowAlloc& A = t->alloc;
        uint8_t* stat = status ? status : A.status_tmp;
        const int64_t nchunks = ceil_div(n, kChunkKeys);
        erase(stat, A.row_tmp);
        hipLaunchKernelGGL(k_chunk_count, dim3(grid_for(nchunks, 4, 1 << 16)), dim3(256), 0, stream, stat, n,
                           (const int64_t*)nullptr, (int)HT_ERASED, A.chunk_cnt, nchunks);
        st = scan_exclusive_i32(A.chunk_cnt, A.chunk_off, nchunks, nullptr, kScanIdentity, 1, A.scan_tmp, stream);
        if (st != HTL_OK) return st;
        hipLaunchKernelGGL(k_erase_push, dim3(grid_for(nchunks, 4, 1 << 16)), dim3(256), 0, stream, stat, A.row_tmp,
                           n, A.chunk_off, A.state, A.free_stack);
        hipLaunchKernelGGL(k_erase_finish, dim3(1), dim3(1), 0, stream, A.state, A.chunk_off + nchunks);
        debug_check_log(t, stream);
        return check_launch("ht_erase");
    }
    erase(status, (int32_t*)nullptr);
    debug_check_log(t, stream);
    return check_launch("ht_erase");
}

htl_status ht_scan(const htl_table* tc, int64_t* keys, uint32_t* last_seen, int32_t* slots,
                   int64_t* n_live_dev, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(tc != nullptr, "ht_scan: null table");
    HTL_REQUIRE(n_live_dev && aligned(n_live_dev, 8), "ht_scan: null or misaligned n_live_dev");
    HTL_REQUIRE(!keys || aligned(keys, 8), "ht_scan: misaligned keys");
    // the export's count / prefix / write passes over every slot: slot
    // order, no shared counter
    htl_table* t = const_cast<htl_table*>(tc);     // only its call temporaries change
    const TableDev& T = t->dev;
    const int64_t nchunks = ceil_div(T.capacity, kExpChunk);
    htl_status st = ensure_exp(t, nchunks);
    if (st != HTL_OK) return st;
    RowAlloc& A = t->alloc;
    const unsigned grid = grid_for(nchunks, 1, 1 << 16);
    hipLaunchKernelGGL(k_exp_count, dim3(grid), dim3(kExpThreads), 0, stream, T, (int64_t)0, T.capacity, nchunks,
                       A.exp_cnt);
    st = scan_exclusive_i32(A.exp_cnt, A.exp_off, nchunks, nullptr, kScanIdentity, 1, A.exp_scan, stream);
    if (st != HTL_OK) return st;
    hipLaunchKernelGGL(k_exp_write, dim3(grid), dim3(kExpThreads), 0, stream, T, (int64_t)0, T.capacity, nchunks,
                       A.exp_off, keys, (void*)nullptr, last_seen, (float*)nullptr, (float*)nullptr, slots);
    hipLaunchKernelGGL(k_exp_total, dim3(1), dim3(1), 0, stream, A.exp_off + nchunks, n_live_dev);
    return check_launch("ht_scan");
}

htl_status ht_export(const htl_table* tc, int64_t slot_begin, int64_t slot_end, int64_t* keys, void* rows,
                     uint32_t* last_seen, float* adam_m, float* adam_v, int64_t* n_dev, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(tc != nullptr, "ht_export: null table");
    htl_table* t = const_cast<htl_table*>(tc);     // only its call temporaries change
    const TableDev& T = t->dev;
    HTL_REQUIRE(slot_begin >= 0 && slot_begin <= slot_end && slot_end <= T.capacity,
                "ht_export: need 0 <= slot_begin <= slot_end <= capacity");
    HTL_REQUIRE(n_dev && aligned(n_dev, 8), "ht_export: null or misaligned n_dev");
    HTL_REQUIRE(!keys || aligned(keys, 8), "ht_export: misaligned keys");
    HTL_REQUIRE(!rows || aligned(rows, ((int64_t)T.dim * T.elem_bytes) % 16 == 0 ? 16 : T.elem_bytes),
                "ht_export: misaligned rows");
    HTL_REQUIRE(!last_seen || T.last_seen, "ht_export: the table keeps no last_seen");
    HTL_REQUIRE((!adam_m && !adam_v) || T.m, "ht_export: the table keeps no Adam state");
    const int64_t nchunks = ceil_div(slot_end - slot_begin, kExpChunk);
    if (nchunks == 0) {
        hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(1), 0, stream, n_dev);
        return check_launch("ht_export");
    }
    htl_status st = ensure_exp(t, ceil_div(T.capacity, kExpChunk));
    if (st != HTL_OK) return st;
    RowAlloc& A = t->alloc;
    const unsigned grid = grid_for(nchunks, 1, 1 << 16);
    hipLaunchKernelGGL(k_exp_count, dim3(grid), dim3(kExpThreads), 0, stream, T, slot_begin, slot_end, nchunks,
                       A.exp_cnt);
    st = scan_exclusive_i32(A.exp_cnt, A.exp_off, nchunks, nullptr, kScanIdentity, 1, A.exp_scan, stream);
    if (st != HTL_OK) return st;
    hipLaunchKernelGGL(k_exp_write, dim3(grid), dim3(kExpThreads), 0, stream, T, slot_begin, slot_end, nchunks,
                       A.exp_off, keys, rows, last_seen, adam_m, adam_v, (int32_t*)nullptr);
    hipLaunchKernelGGL(k_exp_total, dim3(1), dim3(1), 0, stream, A.exp_off + nchunks, n_dev);
    return check_launch("ht_export");
}

htl_status ht_import(htl_table* t, const int64_t* keys, int64_t n, const void* rows, const uint32_t* last_seen,
                     const float* adam_m, const float* adam_v, uint8_t* status, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_import: null table");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "ht_import: n out of range");
    if (n == 0) return HTL_OK;
    const TableDev& T0 = t->dev;
    HTL_REQUIRE(keys && rows && status && aligned(keys, 8), "ht_import: null or misaligned keys/rows/status");
    HTL_REQUIRE(aligned(rows, ((int64_t)T0.dim * T0.elem_bytes) % 16 == 0 ? 16 : T0.elem_bytes),
                "ht_import: misaligned rows");
    HTL_REQUIRE(!last_seen || T0.last_seen, "ht_import: the table keeps no last_seen");
    HTL_REQUIRE((!adam_m && !adam_v) || (adam_m && adam_v && T0.m), "ht_import: Adam state needs both m and v "
                                                                    "and a table that keeps it");
    htl_status st = ensure_tmp(t, n);
    if (st != HTL_OK) return st;
    int32_t* handles = t->alloc.row_tmp;
    const uint32_t keep_step = t->max_step;
    t->log_ok = false;   // last_seen values set from outside: the log no longer covers them
    st = ht_find_or_insert(t, keys, n, nullptr, 0u, handles, status, stream);
    if (st != HTL_OK) return st;
    t->max_step = keep_step;
    const TableDev& T = t->dev;
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    const int64_t items = (row_bytes % 16 == 0) ? n * (row_bytes / 16) : n * T.dim;
    hipLaunchKernelGGL(k_imp_rows, dim3(grid_for(items > n * T.dim ? items : n * T.dim, 256 * 4)), dim3(256), 0,
                       stream, T, n, handles, status, rows, adam_m, adam_v);
    if (last_seen) {
        hipLaunchKernelGGL(k_imp_ls<4>, dim3(grid_for(n, kProbeBlock / 4)), dim3(kProbeBlock), 0, stream, T, keys, n,
                           status, last_seen);
        t->max_step = 0xFFFFFFFFu;       // values unknown on the host: selections check all four digits
    }
    return check_launch("ht_import");
}

htl_status ht_rows(const htl_table* t, const void** rows, int64_t* row_bytes) {
    clear_error();
    HTL_REQUIRE(t, "ht_rows: null table");
    if (rows) *rows = t->dev.rows;
    if (row_bytes) *row_bytes = (int64_t)t->dim * t->dev.elem_bytes;
    return HTL_OK;
}

htl_status ht_access_log_rebuild(htl_table* t, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_access_log_rebuild: null table");
    HTL_REQUIRE(t->log.entries != nullptr, "ht_access_log_rebuild: the table keeps no access log");
    const TableDev& T = t->dev;
    const int64_t M = T.capacity;
    const uint64_t cap = t->log.cap_mask + 1;
    // device temporaries: range [3], per-step counts and cursors [kLogSteps]
    unsigned long long* range = nullptr;
    uint32_t* cnt = nullptr;
    unsigned long long* cursor = nullptr;
    auto release = [&]() {
        if (range) (void)hipFree(range);
        if (cnt) (void)hipFree(cnt);
        if (cursor) (void)hipFree(cursor);
    };
    if (hipMalloc((void**)&range, 3 * sizeof(unsigned long long)) != hipSuccess ||
        hipMalloc((void**)&cnt, (size_t)kLogSteps * 4) != hipSuccess ||
        hipMalloc((void**)&cursor, (size_t)kLogSteps * 8) != hipSuccess) {
        (void)hipGetLastError();
        release();
        return fail(HTL_ERR_NOMEM, "ht_access_log_rebuild: temporaries allocation failed");
    }
    const unsigned long long init[3] = {0xFFFFFFFFull, 0ull, 0ull};
    unsigned long long host[3] = {0, 0, 0};
    htl_status st = HTL_OK;
    auto hip = [&](hipError_t e, const char* what) {
        if (st == HTL_OK && e != hipSuccess) st = fail(HTL_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    };
    hip(hipMemcpyAsync(range, init, sizeof(init), hipMemcpyHostToDevice, stream), "ht_access_log_rebuild: copy");
    if (st == HTL_OK)
        hipLaunchKernelGGL(k_log_range, dim3(grid_for(M, 256 * 16, 2048)), dim3(256), 0, stream, T.last_seen, M, range);
    hip(hipMemcpyAsync(host, range, sizeof(host), hipMemcpyDeviceToHost, stream), "ht_access_log_rebuild: copy");
    hip(hipStreamSynchronize(stream), "ht_access_log_rebuild: synchronize");
    if (st != HTL_OK) {
        release();
        return st;
    }
    const uint32_t lo = (uint32_t)host[0], hi = (uint32_t)host[1];
    const uint64_t live = host[2];
    if (live == 0) {                          // nothing live: an empty log
        release();
        st = log_reset(t, stream);
        if (st == HTL_OK && t->max_step == 0xFFFFFFFFu) t->max_step = 0u;
        return st;
    }
    if ((int64_t)(hi - lo) >= kLogSteps || live > cap) {
        release();
        return fail(HTL_ERR_INVALID, "ht_access_log_rebuild: the live keys' last_seen span 4096 steps or more, or "
                                     "they outnumber the ring's entries; the eviction choice keeps scanning");
    }
    const int64_t span = (int64_t)(hi - lo) + 1;
    std::vector<uint32_t> hc(span);
    std::vector<unsigned long long> hcur(kLogSteps, 0ull);
    std::vector<LogSeg> segs(kLogSteps);
    for (auto& g : segs) g = LogSeg{0xFFFFFFFFu, 0u, 0ull, 0ull};
    hip(hipMemsetAsync(cnt, 0, (size_t)kLogSteps * 4, stream), "ht_access_log_rebuild: clear");
    const unsigned gfill = grid_for(M, 256 * 64, 1024);
    if (st == HTL_OK)
        hipLaunchKernelGGL(k_log_fill, dim3(gfill), dim3(256), 0, stream, T.last_seen, M, lo, cnt,
                           (unsigned long long*)nullptr, t->log.entries, t->log.cap_mask);
    hip(hipMemcpyAsync(hc.data(), cnt, (size_t)span * 4, hipMemcpyDeviceToHost, stream), "ht_access_log_rebuild: copy");
    hip(hipStreamSynchronize(stream), "ht_access_log_rebuild: synchronize");
    if (st != HTL_OK) {
        release();
        return st;
    }
    // the steps' runs in step order from ring position 0
    uint64_t at = 0;
    uint32_t s_min = lo;
    bool first = true;
    for (int64_t b = 0; b < span; ++b) {
        if (!hc[b]) continue;
        const uint32_t s = lo + (uint32_t)b;
        if (first) {
            s_min = s;
            first = false;
        }
        hcur[b] = at;
        segs[s & kLogStepMask] = LogSeg{s, 0u, at, at + hc[b]};
        at += hc[b];
    }
    hip(hipMemcpyAsync(cursor, hcur.data(), (size_t)kLogSteps * 8, hipMemcpyHostToDevice, stream),
        "ht_access_log_rebuild: copy");
    hip(hipMemcpyAsync(t->log.segs, segs.data(), (size_t)kLogSteps * sizeof(LogSeg), hipMemcpyHostToDevice, stream),
        "ht_access_log_rebuild: copy");
    hip(hipMemsetAsync(t->log.cnt, 0, (size_t)kLogSteps * kLogSubs * kLogCntStride * 8, stream),
        "ht_access_log_rebuild: clear");
    if (st == HTL_OK) {
        hipLaunchKernelGGL(k_log_fill, dim3(gfill), dim3(256), 0, stream, T.last_seen, M, lo, cnt, cursor,
                           t->log.entries, t->log.cap_mask);
        hipLaunchKernelGGL(k_log_set, dim3(grid_for(span, 256, 16)), dim3(256), 0, stream, t->log.cnt, cnt, lo, span,
                           t->log.st, t->log_par, (uint64_t)live, s_min);
        st = check_launch("ht_access_log_rebuild");
    }
    hip(hipStreamSynchronize(stream), "ht_access_log_rebuild: synchronize");
    release();
    if (st != HTL_OK) return st;
    t->log_ok = true;
    t->log_first = false;
    t->erase_pending = false;
    if (t->max_step == 0xFFFFFFFFu || t->max_step < hi) t->max_step = hi;
    return HTL_OK;
}

htl_status ht_access_log_state(const htl_table* t, int64_t* out_dev, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t && out_dev && aligned(out_dev, 8), "ht_access_log_state: null or misaligned argument");
    HTL_REQUIRE(t->log.entries != nullptr, "ht_access_log_state: the table keeps no access log");
    hipLaunchKernelGGL(k_log_state, dim3(1), dim3(1), 0, stream, t->log.st, t->log_par, t->log_ok ? 1 : 0, out_dev);
    return check_launch("ht_access_log_state");
}

htl_status ht_view(const htl_table* t, htl_view* out) {
    clear_error();
    HTL_REQUIRE(t && out, "ht_view: null argument");
    out->capacity = t->dev.capacity;
    out->dim = t->dim;
    out->dtype = t->dtype;
    out->keys = t->dev.keys;
    out->rows = t->dev.rows;
    out->last_seen = t->dev.last_seen;
    out->adam_m = t->dev.m;
    out->adam_v = t->dev.v;
    out->row_of_slot = t->dev.rowid;
    return HTL_OK;
}

}  // extern "C"
