// Eviction choice for an online table: the floor(live * num / den) live keys
// that are smallest by (last_seen, key).
//
// MTGenRec (arXiv 2505.12663), Abstract: embeddings are inserted and deleted
// in real time; MTGR (arXiv 2505.18654) section 5, "Embedding Management":
// every key carries metadata and live keys can be scanned compactly.  The
// pages name no eviction policy; least recently used, ties broken by the key
// value, is this library's.
//
// All on the device, no host synchronisation and no counter atomics (a
// counter that every block bumps serialises on MI355X):
//   collect -- the table is cut into chunks of kChunk slots; each chunk
//              compacts its live slots' (last_seen, slot) into its own fixed
//              region of the candidate arrays and records its count and its
//              largest last_seen.  Only last_seen is read (dead slots hold
//              kLsDead there), so the pass moves 4 bytes per slot, not 12;
//              keys are read later, through the slot, for the candidates
//              that tie on the selected last_seen and for the victims;
//   init    -- one block sums the counts (live L), takes the maximum
//              last_seen and sets k = floor(L * num / den);
//   select  -- the cut last_seen by radix select with 8-bit digits: per
//              digit, LDS histograms of the candidates that match the digits
//              chosen so far (a persistent grid, so each of the 256 global
//              bins, one cache line apart, gets one add per block), then one
//              block scans the bins for the bucket holding the k-th smallest
//              (only as many digits as the largest last_seen needs).  Then
//              the cut key among the candidates that tie on last_seen (keys
//              with the sign bit flipped, so unsigned order is signed order),
//              compacted per chunk: one histogram of a 12-bit window that
//              starts at the highest bit in which the ties differ (their
//              AND and OR say which), in LDS per block and then 4096 global
//              bins; a one-block pick of the bucket that holds the cut; the
//              ties in that bucket gathered (and compacted in place); and
//              one block that ranks them in LDS (at most kFinalCap of them:
//              uniform keys leave about ties / 4096) or, for a larger
//              bucket (keys that share more high bits, such as a table id
//              over small ids), takes the bits below the window by 8-bit
//              radix passes of its own.
//              Every launch here costs a few microseconds even with little
//              to do, so the passes are few.  (A pick fused into the
//              histogram pass by a last-block ticket needs a device-scope
//              fence per block, which writes back L2 on this multi-die part
//              and cost far more than the extra launch.)
//   emit    -- victims (candidates at or below the selected (last_seen,
//              key)) are counted per chunk, the counts prefix-summed, and
//              written densely.
// Every pass after the collect takes one chunk per wave, with wave-wide
// prefixes: no block barrier per chunk.
#include "htl_common.h"

namespace htl {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;               // table slots per chunk (one block pass)
constexpr int kPerThread = kChunk / kThreads;
// persistent grid of the histogram passes (selection on the online
// workload: 512 blocks 0.383 ms, 1024 0.364 ms, 4096 0.452 ms)
constexpr int kHistBlocks = 1024;
constexpr int kBinStride = 32;             // words between global histogram bins

struct LruState {
    int64_t n_live;
    int64_t k;            // victims wanted
    int64_t k_rem;        // rank (1-based) still to find inside the current last_seen prefix
    int64_t k_tie;        // rank (1-based) of the cut among the ties, then inside the key prefix
    uint32_t ls_cut;      // the cut last_seen (set by k_lru_ties)
    uint32_t pad3;
    uint32_t ls_max;
    uint32_t ls_digits;   // last_seen digits in use
    uint32_t ls_prefix;   // selected last_seen (complete after its last digit)
    uint32_t pad;
    uint64_t key_prefix;  // selected biased key
    unsigned long long key_and, key_or;   // over the biased keys of the ties
    int32_t mode;         // kModeLog: candidates from the access log (set by k_lru_log_init)
    int32_t ksel_state;   // cut key: 0 histogram pending, 1 final rank pending, 2 known
    int32_t ksel_fix;     // bits >= ksel_fix of key_prefix are fixed
    int32_t ksel_n;       // keys gathered for the final rank
    uint64_t win_begin, win_end;          // ring window of the log's candidates
    uint32_t hist[256 * kBinStride];
};

constexpr int kModeScan = 0;
constexpr int kModeLog = 1;
constexpr int kKeyWin = 12;            // bits of the cut-key histogram window
constexpr int kKeyBins = 1 << kKeyWin;
constexpr int kFinalCap = 4096;        // keys the final rank holds in LDS

// Chunks that can hold candidates: all of them, or with the access log the
// window's (the later ones have none).
__device__ __forceinline__ int64_t busy_chunks(const struct LruState* st, int64_t nchunks, int use_log, int log_chunk) {
    if (!use_log || st->mode != kModeLog) return nchunks;
    const int64_t nw = (int64_t)(st->win_end - st->win_begin + (uint64_t)log_chunk - 1) / log_chunk;
    return nw < nchunks ? nw : nchunks;
}


struct LruWs {
    LruState* st;
    uint32_t* cand_ls;     // [nchunks * kChunk]: per chunk, its live slots' last_seen first
    uint32_t* cand_slot;   // [nchunks * kChunk]: those slots
    uint64_t* ties;        // [nchunks * kChunk]: per chunk, candidates tying on last_seen
    int32_t* chunk_cnt;    // [nchunks]
    uint32_t* chunk_max;   // [nchunks]
    int32_t* tie_cnt;      // [nchunks]
    int32_t* vic_cnt;      // [nchunks]
    int32_t* vic_off;      // [nchunks + 1]
    uint32_t* khist;       // [kKeyBins]: cut-key histogram
    uint64_t* sel;         // [kFinalCap]: ties of the cut bucket
    int64_t nchunks;
    size_t bytes;
};

LruWs lru_layout(int64_t M, char* base) {
    LruWs w{};
    w.nchunks = ceil_div(M, kChunk);
    const size_t cap = (size_t)w.nchunks * kChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.st = (LruState*)take(sizeof(LruState));
    w.cand_ls = (uint32_t*)take(cap * 4);
    w.cand_slot = (uint32_t*)take(cap * 4);
    w.ties = (uint64_t*)take(cap * 8);
    w.chunk_cnt = (int32_t*)take((size_t)w.nchunks * 4);
    w.chunk_max = (uint32_t*)take((size_t)w.nchunks * 4);
    w.tie_cnt = (int32_t*)take((size_t)w.nchunks * 4);
    w.vic_cnt = (int32_t*)take((size_t)w.nchunks * 4);
    w.vic_off = (int32_t*)take((size_t)(w.nchunks + 1) * 4);
    w.khist = (uint32_t*)take((size_t)kKeyBins * 4);
    w.sel = (uint64_t*)take((size_t)kFinalCap * 8);
    w.bytes = off;
    return w;
}

__device__ __forceinline__ uint64_t bias(int64_t k) { return (uint64_t)k ^ 0x8000000000000000ull; }

// Block-wide exclusive prefix of v over thread order; returns the total.
__device__ __forceinline__ int block_prefix(int& v, int* s_wave) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave[wid] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const int c = s_wave[w];
        before += (w < wid) ? c : 0;
        tot += c;
    }
    __syncthreads();
    v = before + incl - v;
    return tot;
}

// Each chunk compacts its live slots (last_seen, slot) into its own region
// (order within the region: by thread, then by the thread's slots), staged
// in LDS.  Only
// last_seen is read: a slot without a live key holds kLsDead there.  Loads
// are 16 bytes per lane: slot quad j * kThreads + tid of the chunk belongs to
// thread tid.
typedef uint32_t u32x4l __attribute__((ext_vector_type(4)));
constexpr int kQuads = kPerThread / 4;

//
// With the access log serving (mode kModeLog), chunk c is instead entries
// [c * E, (c + 1) * E) of the ring window (E = log_chunk <= kChunk: the ring
// holds at most nchunks * E entries): an entry is a candidate iff its step
// is at most the cut step and last_seen of its slot still equals that step;
// chunks past the window are neither written nor read by the passes after
// (they stop at the window's chunks).  E below kChunk spreads the window's
// candidates over more chunks, so the passes that take one chunk per wave
// have more waves at work.  An entry found stale is overwritten with
// kLogNoSlot: it can never be current again (its slot's last_seen only
// moves to later steps, or the key is erased, and a slot freed and claimed
// again within one step ends the log), and the oldest steps' entries, most
// of them stale, are read again by every selection until their last live
// key goes -- this way without a last_seen read each.
__global__ __launch_bounds__(kThreads) void k_lru_collect(TableDev T, int64_t nchunks,
                                                         uint32_t* __restrict__ cand_ls,
                                                         uint32_t* __restrict__ cand_slot,
                                                         int32_t* __restrict__ chunk_cnt,
                                                         uint32_t* __restrict__ chunk_max, int use_log, LogDev L,
                                                         const LruState* __restrict__ st, int log_chunk) {
    __shared__ int s_wave[kThreads / 64];
    __shared__ uint32_t s_max[kThreads / 64];
    __shared__ uint32_t s_ls[kChunk];
    __shared__ uint16_t s_off[kChunk];
    const int tid = threadIdx.x;
    if (use_log && st->mode == kModeLog) {
        const uint64_t wb = st->win_begin;
        const int64_t W = (int64_t)(st->win_end - wb);
        const uint32_t thr = st->ls_prefix;
        const int64_t nb = busy_chunks(st, nchunks, use_log, log_chunk);   // chunks past them are not read
        for (int64_t c = blockIdx.x; c < nb; c += gridDim.x) {
            const int64_t e0 = c * log_chunk;    // window entry of the chunk's first
            const int64_t r0 = c * kChunk;       // the chunk's candidate region
            uint64_t ent[kPerThread];
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                const int64_t e = e0 + j * kThreads + tid;
                ent[j] = (j * kThreads + tid < log_chunk && e < W) ? L.entries[(wb + (uint64_t)e) & L.cap_mask]
                                                                   : ~0ull;
            }
            uint32_t now[kPerThread];
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                const uint32_t slot = (uint32_t)ent[j], step = (uint32_t)(ent[j] >> 32);
                // (slot < capacity always holds for entries the table wrote; the
                // test keeps every read in bounds regardless)
                now[j] = (slot != kLogNoSlot && (int64_t)slot < T.capacity && step <= thr) ? T.last_seen[slot]
                                                                                           : kLsDead;
            }
            uint32_t live = 0;
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                const uint32_t slot = (uint32_t)ent[j];
                if (now[j] != kLsDead && now[j] == (uint32_t)(ent[j] >> 32)) live |= 1u << j;
                else if (slot != kLogNoSlot && (int64_t)slot < T.capacity && (uint32_t)(ent[j] >> 32) <= thr)
                    // read, and stale
                    L.entries[(wb + (uint64_t)(e0 + j * kThreads + tid)) & L.cap_mask] =
                        (ent[j] & 0xFFFFFFFF00000000ull) | kLogNoSlot;
            }
            int pos = __popc(live);
            const int total = block_prefix(pos, s_wave);
            uint32_t my_max = 0;
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                if (live & (1u << j)) {
                    my_max = now[j] > my_max ? now[j] : my_max;
                    s_ls[pos] = now[j];
                    s_off[pos] = (uint16_t)(j * kThreads + tid);
                    ++pos;
                }
            }
            for (int off = 32; off > 0; off >>= 1) {
                const uint32_t y = __shfl_xor(my_max, off);
                my_max = y > my_max ? y : my_max;
            }
            if (lane_id() == 0) s_max[tid >> 6] = my_max;
            __syncthreads();
            for (int j = tid; j < total; j += kThreads) {
                cand_ls[r0 + j] = s_ls[j];
                // the entry again (just read by this block): its slot
                cand_slot[r0 + j] = (uint32_t)L.entries[(wb + (uint64_t)(e0 + s_off[j])) & L.cap_mask];
            }
            if (tid == 0) {
                uint32_t m = 0;
                for (int w = 0; w < kThreads / 64; ++w) m = s_max[w] > m ? s_max[w] : m;
                chunk_cnt[c] = total;
                chunk_max[c] = m;
            }
            __syncthreads();
        }
        return;
    }
    const u32x4l* ls4 = reinterpret_cast<const u32x4l*>(T.last_seen);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t qbase = c * (kChunk / 4);           // first slot quad of the chunk
        uint32_t ls[kPerThread];
        uint32_t live = 0;                                // bit 4j+e: slot 4*(quad j)+e
#pragma unroll
        for (int j = 0; j < kQuads; ++j) {
            const int64_t q = qbase + (int64_t)j * kThreads + tid;
            u32x4l x;
            x.x = x.y = x.z = x.w = kLsDead;
            // capacity is a multiple of 4 or below 4 slots
            if (4 * q + 3 < T.capacity) {
                x = ls4[q];
            } else if (4 * q < T.capacity) {
                x.x = T.last_seen[4 * q];
                if (4 * q + 1 < T.capacity) x.y = T.last_seen[4 * q + 1];
            }
            ls[4 * j] = x.x;
            ls[4 * j + 1] = x.y;
            ls[4 * j + 2] = x.z;
            ls[4 * j + 3] = x.w;
        }
#pragma unroll
        for (int e = 0; e < kPerThread; ++e)
            if (ls[e] != kLsDead) live |= 1u << e;
        int pos = __popc(live);
        const int total = block_prefix(pos, s_wave);
        uint32_t my_max = 0;
        const int64_t base = 4 * qbase;
        // compacted in LDS first: the global stores then go out dense, a
        // few per block, instead of many sparse partial-line stores
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
            if (live & (1u << e)) {
                my_max = ls[e] > my_max ? ls[e] : my_max;
                s_ls[pos] = ls[e];
                s_off[pos] = (uint16_t)(4 * ((e >> 2) * kThreads + tid) + (e & 3));
                ++pos;
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const uint32_t y = __shfl_xor(my_max, off);
            my_max = y > my_max ? y : my_max;
        }
        if (lane_id() == 0) s_max[tid >> 6] = my_max;
        __syncthreads();
        for (int j = tid; j < total; j += kThreads) {
            cand_ls[base + j] = s_ls[j];
            cand_slot[base + j] = (uint32_t)(base + s_off[j]);
        }
        if (tid == 0) {
            uint32_t m = 0;
            for (int w = 0; w < kThreads / 64; ++w) m = s_max[w] > m ? s_max[w] : m;
            chunk_cnt[c] = total;
            chunk_max[c] = m;
        }
        __syncthreads();
    }
}

// Live keys of step s: the sum of its partial counts (none if the record is
// another step's: that step has no live key left, its counts are zero).
__device__ __forceinline__ int64_t log_count(const LogDev& L, uint32_t s) {
    if (L.segs[s & kLogStepMask].step != s) return 0;
    const int64_t* c = L.cnt + (int64_t)(s & kLogStepMask) * kLogSubs * kLogCntStride;
    int64_t sum = 0;
#pragma unroll 8
    for (int q = 0; q < kLogSubs; ++q) sum += c[q * kLogCntStride];
    return sum;
}

// One block, first, on a table with an access log.  If the log serves:
// the live count from the step counts of [s_min, s_now], k, and the cut
// step s* (the last_seen of the k-th smallest key): every live key with
// last_seen < s* is a victim, and k_rem of those with last_seen == s*, by
// key.  All their entries lie in the ring window [tail, end of s*).  The
// last_seen digits are then known (ls_digits = 0: their passes skip), and
// s_min and the tail move up to the oldest step that has live keys.  If
// the log does not serve, the scan path runs (mode kModeScan).
__global__ __launch_bounds__(1024) void k_lru_log_init(LruState* st, LogDev L, int par, uint32_t s_now, int64_t num,
                                                      int64_t den) {
    __shared__ long long s_sum[1024 / 64];
    __shared__ uint32_t s_first[1024 / 64];
    LogState* ls = L.st;
    const uint32_t s0 = ls->s_min;
    const int64_t span = (int64_t)(s_now - s0) + 1;
    if (ls->bad || s_now < s0 || span > kLogSteps) {     // the same in every thread
        if (threadIdx.x == 0) st->mode = kModeScan;
        return;
    }
    const int64_t per = (span + 1023) / 1024;
    const int64_t a = threadIdx.x * per;
    const int64_t b = a + per < span ? a + per : span;
    long long sum = 0;
    uint32_t first = 0xFFFFFFFFu;
    for (int64_t j = a; j < b; ++j) {
        const int64_t c = log_count(L, s0 + (uint32_t)j);
        sum += c;
        if (c > 0 && first == 0xFFFFFFFFu) first = s0 + (uint32_t)j;
    }
    // exclusive prefix of the per-thread sums (steps in thread order), total,
    // and the first step with live keys
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    long long incl = sum;
    uint32_t fmin = first;
    for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
        const uint32_t f = __shfl_xor(fmin, off);
        fmin = f < fmin ? f : fmin;
    }
    if (lane == 63) s_sum[wid] = incl;
    if (lane == 0) s_first[wid] = fmin;
    if (threadIdx.x < 256) st->hist[threadIdx.x * kBinStride] = 0u;
    __syncthreads();
    long long before = incl - sum, total = 0;
    uint32_t fl = 0xFFFFFFFFu;
    for (int w = 0; w < 1024 / 64; ++w) {
        before += w < wid ? s_sum[w] : 0;
        total += s_sum[w];
        fl = s_first[w] < fl ? s_first[w] : fl;
    }
    const int64_t k = ((int64_t)total * num) / den;
    if (k > 0 && before < k && k <= before + sum) {
        long long cum = before;
        for (int64_t j = a; j < b; ++j) {
            const uint32_t s = s0 + (uint32_t)j;
            const int64_t c = log_count(L, s);
            if (cum + c >= k) {
                st->ls_prefix = s;
                st->k_rem = k - cum;
                st->win_end = L.segs[s & kLogStepMask].end;
                break;
            }
            cum += c;
        }
    }
    if (threadIdx.x == 0) {
        const uint64_t tail = fl != 0xFFFFFFFFu ? L.segs[fl & kLogStepMask].begin : ls->head[par];
        ls->s_min = fl != 0xFFFFFFFFu ? fl : s_now;
        ls->tail = tail;
        st->win_begin = tail;
        st->n_live = (int64_t)total;
        st->k = k;
        st->ls_max = s_now;
        st->ls_digits = 0u;
        st->key_prefix = 0ull;
        st->key_and = ~0ull;
        st->key_or = 0ull;
        st->ksel_state = 0;
        st->mode = kModeLog;
        if (k <= 0) {
            st->k_rem = 0;
            st->ls_prefix = 0u;
            st->win_end = tail;
        }
    }
}

// One block: live count, maximum last_seen, k, and a cleared histogram
// (the scan path; with the log serving, k_lru_log_init has set them).
__global__ __launch_bounds__(1024) void k_lru_init(LruState* st, const int32_t* __restrict__ chunk_cnt,
                                                  const uint32_t* __restrict__ chunk_max, int64_t nchunks,
                                                  int64_t num, int64_t den, int use_log) {
    if (use_log && st->mode == kModeLog) return;
    __shared__ unsigned long long s_sum[1024 / 64];
    __shared__ uint32_t s_max[1024 / 64];
    unsigned long long sum = 0;
    uint32_t mx = 0;
    // kInitUnroll independent loads of each array in flight per thread
    constexpr int kInitUnroll = 8;
    for (int64_t c0 = threadIdx.x; c0 < nchunks; c0 += (int64_t)blockDim.x * kInitUnroll) {
        int32_t cv[kInitUnroll];
        uint32_t mv[kInitUnroll];
#pragma unroll
        for (int u = 0; u < kInitUnroll; ++u) {
            const int64_t c = c0 + (int64_t)u * blockDim.x;
            cv[u] = c < nchunks ? chunk_cnt[c] : 0;
            mv[u] = c < nchunks ? chunk_max[c] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kInitUnroll; ++u) {
            sum += (unsigned long long)cv[u];
            mx = mv[u] > mx ? mv[u] : mx;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        sum += __shfl_xor(sum, off);
        const uint32_t y = __shfl_xor(mx, off);
        mx = y > mx ? y : mx;
    }
    if (lane_id() == 0) {
        s_sum[threadIdx.x >> 6] = sum;
        s_max[threadIdx.x >> 6] = mx;
    }
    if (threadIdx.x < 256) st->hist[threadIdx.x * kBinStride] = 0u;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long L = 0;
        uint32_t m = 0;
        for (int w = 0; w < 1024 / 64; ++w) {
            L += s_sum[w];
            m = s_max[w] > m ? s_max[w] : m;
        }
        st->n_live = (int64_t)L;
        st->k = ((int64_t)L * num) / den;
        st->k_rem = st->k;
        st->ls_max = m;
        uint32_t d = 1;
        while (d < 4 && (m >> (8 * d)) != 0u) ++d;
        st->ls_digits = d;
        st->ls_prefix = 0u;
        st->key_prefix = 0ull;
        st->key_and = ~0ull;
        st->key_or = 0ull;
        st->ksel_state = 0;
    }
}

// A block's LDS histogram (s_h, 256 bins, complete) is added into the
// global one; the bins sit kBinStride words apart, one cache line each, so
// that the blocks' atomics spread over the L2 channels.
__device__ __forceinline__ void commit_hist(LruState* st, const uint32_t* s_h) {
    const uint32_t c = s_h[threadIdx.x];
    if (c) atomicAdd(&st->hist[threadIdx.x * kBinStride], c);
}

// One block of 256 threads after each last_seen digit's histogram: a
// block-wide scan of the 256 bins finds the bucket that holds rank k_rem;
// the prefix is narrowed and the histogram cleared for the next digit.
__global__ __launch_bounds__(256) void k_lru_pick(LruState* st, int d) {
    __shared__ int64_t s_wave[4];
    const int t = threadIdx.x, lane = lane_id(), wid = t >> 6;
    const bool active = st->k > 0 && (uint32_t)d < st->ls_digits;
    const int64_t rem = st->k_rem;                // read before any thread may update it
    const int64_t c = st->hist[t * kBinStride];
    st->hist[t * kBinStride] = 0u;
    int64_t incl = c;
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave[wid] = incl;
    __syncthreads();
    for (int w = 0; w < wid; ++w) incl += s_wave[w];
    const int64_t excl = incl - c;
    if (active && excl < rem && (incl >= rem || t == 255)) {
        st->k_rem = rem - excl;
        st->ls_prefix |= (uint32_t)t << (8 * d);
    }
}

// Calls f(c, cnt) for each chunk c = w + i * W whose count is nonzero, where
// w is this wave's index in the grid and W the number of waves: each wave
// works through its own chunks, so the per-chunk work needs no block
// barrier.  The wave's counts are loaded 64 at a time in one round (a chain
// of one dependent load per chunk costs microseconds once the lists are
// sparse).  When zero_out is given, zero_out[c] = 0 is stored for the
// chunks skipped.  f may use wave-wide operations: cnt is wave-uniform.
template <class F>
__device__ __forceinline__ void for_wave_chunks(const int32_t* __restrict__ cnts, int64_t nchunks,
                                                int32_t* __restrict__ zero_out, F&& f) {
    constexpr int kWaves = kThreads / 64;
    const int lane = lane_id();
    const int64_t W = (int64_t)gridDim.x * kWaves;
    const int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t mine = nchunks > w ? (nchunks - w + W - 1) / W : 0;
    for (int64_t i0 = 0; i0 < mine; i0 += 64) {
        const int64_t i = i0 + lane;
        int32_t cnt = 0;
        if (i < mine) {
            cnt = cnts[w + i * W];
            if (cnt <= 0 && zero_out) zero_out[w + i * W] = 0;
        }
        const int nb = (int)(mine - i0 < 64 ? mine - i0 : 64);
        for (int j = 0; j < nb; ++j) {
            const int c = __shfl(cnt, j);
            if (c > 0) f(w + (i0 + j) * W, c);
        }
    }
}

// last_seen digit d over the candidates matching the higher digits.
__global__ __launch_bounds__(kThreads) void k_lru_hist_ls(LruState* __restrict__ st,
                                                         const uint32_t* __restrict__ cand_ls,
                                                         const int32_t* __restrict__ chunk_cnt, int64_t nchunks,
                                                         int d) {
    if ((uint32_t)d >= st->ls_digits || st->k <= 0) return;
    __shared__ uint32_t s_h[256];
    s_h[threadIdx.x] = 0u;
    __syncthreads();
    const uint32_t hi_shift = 8u * (uint32_t)(d + 1);
    const uint32_t want = hi_shift >= 32 ? 0u : (st->ls_prefix >> hi_shift);
    const int lane = lane_id();
    for_wave_chunks(chunk_cnt, nchunks, nullptr, [&](int64_t c, int cnt) {
        for (int j = lane; j < cnt; j += 64) {
            const uint32_t x = cand_ls[c * kChunk + j];
            const uint32_t hi = hi_shift >= 32 ? 0u : (x >> hi_shift);
            if (hi == want) atomicAdd(&s_h[(x >> (8 * d)) & 255u], 1u);
        }
    });
    __syncthreads();
    commit_hist(st, s_h);
}

// Candidates tying on the cut last_seen, compacted per chunk, with their
// keys (read through the slot), and the AND and OR of all their keys (the
// highest bit where the two differ is where the cut-key window starts).
// Every block first takes the pick of the last last_seen digit from the 256
// histogram bins itself (the same in every block; block 0 records it in
// ls_cut and k_tie, fields no other block reads here), which saves the
// launch of a one-block pick; with the access log serving, the cut is
// already known.  Also clears the cut-key histogram.
__global__ __launch_bounds__(kThreads) void k_lru_ties(LruState* __restrict__ st,
                                                      const uint32_t* __restrict__ cand_ls,
                                                      const uint32_t* __restrict__ cand_slot,
                                                      const int64_t* __restrict__ keys,
                                                      const int32_t* __restrict__ chunk_cnt, int64_t nchunks,
                                                      uint64_t* __restrict__ ties, int32_t* __restrict__ tie_cnt,
                                                      uint32_t* __restrict__ khist, int use_log, int log_chunk) {
    __shared__ unsigned long long s_and[kThreads / 64], s_or[kThreads / 64];
    __shared__ int64_t s_wv[kThreads / 64];
    __shared__ uint32_t s_thr;
    __shared__ int64_t s_rem;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < kKeyBins; i += (int64_t)gridDim.x * kThreads)
        khist[i] = 0u;
    const int64_t nb = busy_chunks(st, nchunks, use_log, log_chunk);
    if (st->k <= 0) {
        for (int64_t c = blockIdx.x * (int64_t)kThreads + threadIdx.x; c < nb; c += (int64_t)gridDim.x * kThreads)
            tie_cnt[c] = 0;
        return;
    }
    const int lane = lane_id();
    {
        // the cut last_seen: the last digit's bucket (kThreads == 256 bins)
        const int64_t rem = st->k_rem;
        const uint32_t pre = st->ls_prefix;
        if (threadIdx.x == 0) {
            s_thr = pre;
            s_rem = rem;
        }
        if (st->ls_digits > 0) {
            const int t = threadIdx.x, wid = t >> 6;
            const int64_t c = st->hist[t * kBinStride];
            int64_t incl = c;
            for (int off = 1; off < 64; off <<= 1) {
                const int64_t y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            if (lane == 63) s_wv[wid] = incl;
            __syncthreads();
            for (int w = 0; w < wid; ++w) incl += s_wv[w];
            const int64_t excl = incl - c;
            if (excl < rem && (incl >= rem || t == 255)) {
                s_thr = pre | (uint32_t)t;
                s_rem = rem - excl;
            }
        }
        __syncthreads();
    }
    const uint32_t thr = s_thr;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->ls_cut = thr;
        st->k_tie = s_rem;
    }
    unsigned long long k_and = ~0ull, k_or = 0ull;
    for_wave_chunks(chunk_cnt, nb, tie_cnt, [&](int64_t c, int cnt) {
        int run = 0;
        for (int j0 = 0; j0 < cnt; j0 += 64) {
            const int j = j0 + lane;
            uint32_t ls = 0, slot = 0;
            if (j < cnt) {
                ls = cand_ls[c * kChunk + j];
                slot = cand_slot[c * kChunk + j];
            }
            const bool tie = j < cnt && ls == thr;
            uint64_t key = 0;
            if (tie) {
                key = bias(keys[slot]);
                k_and &= key;
                k_or |= key;
            }
            const uint64_t m = __ballot(tie);
            if (tie) ties[c * kChunk + run + __popcll(m & lanemask_lt())] = key;
            run += __popcll(m);
        }
        if (lane == 0) tie_cnt[c] = run;
    });
    for (int off = 32; off > 0; off >>= 1) {
        k_and &= __shfl_xor(k_and, off);
        k_or |= __shfl_xor(k_or, off);
    }
    if (lane == 0) {
        s_and[threadIdx.x >> 6] = k_and;
        s_or[threadIdx.x >> 6] = k_or;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w) {
            k_and &= s_and[w];
            k_or |= s_or[w];
        }
        if (k_and != ~0ull) atomicAnd(&st->key_and, k_and);
        if (k_or != 0ull) atomicOr(&st->key_or, k_or);
    }
}

// The cut-key window: bits [lo, fix) of the biased key, where fix is one
// past the highest bit in which the ties differ (they all agree above it).
__device__ __forceinline__ void ksel_window(const LruState* st, int& fix, int& lo) {
    const uint64_t diff = st->key_and ^ st->key_or;
    fix = diff ? 64 - __clzll((long long)diff) : 0;
    lo = fix > kKeyWin ? fix - kKeyWin : 0;
}

// Does a key match the bits >= fix of the prefix?
__device__ __forceinline__ bool ksel_match(uint64_t key, uint64_t prefix, int fix) {
    return fix >= 64 || (key >> fix) == (prefix >> fix);
}

// Histogram of the ties' window digits: LDS bins per block (a chunk per
// wave), the nonzero ones then added to the global bins.
__global__ __launch_bounds__(kThreads) void k_lru_hist_key(const LruState* __restrict__ st,
                                                          const uint64_t* __restrict__ ties,
                                                          const int32_t* __restrict__ tie_cnt, int64_t nchunks,
                                                          uint32_t* __restrict__ khist, int use_log, int log_chunk) {
    __shared__ uint32_t s_h[kKeyBins];
    if (st->k <= 0) return;
    const int64_t nb = busy_chunks(st, nchunks, use_log, log_chunk);
    int fix, lo;
    ksel_window(st, fix, lo);
    if (fix == 0) return;                      // one tie: nothing to count
    for (int b = threadIdx.x; b < kKeyBins; b += kThreads) s_h[b] = 0u;
    __syncthreads();
    const uint64_t mask = (1ull << (fix - lo)) - 1ull;
    const int lane = lane_id();
    for_wave_chunks(tie_cnt, nb, nullptr, [&](int64_t c, int cnt) {
        for (int j = lane; j < cnt; j += 64) atomicAdd(&s_h[(uint32_t)((ties[c * kChunk + j] >> lo) & mask)], 1u);
    });
    __syncthreads();
    for (int b = threadIdx.x; b < kKeyBins; b += kThreads)
        if (s_h[b]) atomicAdd(&khist[b], s_h[b]);
}

// Block-wide inclusive scan over 1024 threads of one count each; s_w holds
// 16 partial sums.  Returns the inclusive prefix of this thread.
__device__ __forceinline__ int64_t scan1024(int64_t v, int64_t* s_w) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int64_t incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_w[wid] = incl;
    __syncthreads();
    for (int w = 0; w < wid; ++w) incl += s_w[w];
    __syncthreads();
    return incl;
}

// One block: the bucket of the window that holds rank k_rem among the ties
// (four bins per thread); its digit joins the prefix.  Done when the window
// reaches bit 0, else the bucket's ties are ranked next.
__global__ __launch_bounds__(1024) void k_lru_pick_key(LruState* st, const uint32_t* __restrict__ khist) {
    __shared__ int64_t s_w[1024 / 64];
    if (st->k <= 0) return;
    int fix, lo;
    ksel_window(st, fix, lo);
    const int t = threadIdx.x;
    if (fix == 0) {                            // a single tie: it is the cut key
        if (t == 0) {
            st->key_prefix = st->key_and;
            st->ksel_state = 2;
        }
        return;
    }
    const int nbins = 1 << (fix - lo);
    const int64_t rem = st->k_tie;
    const uint64_t base = st->key_and & ~((fix >= 64 ? 0ull : (1ull << fix)) - 1ull);
    static_assert(kKeyBins == 4 * 1024, "four bins per thread");
    uint32_t v[4];
    int64_t c = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v[u] = 4 * t + u < nbins ? khist[4 * t + u] : 0u;
        c += v[u];
    }
    const int64_t incl = scan1024(c, s_w);
    int64_t run = incl - c;
    if (run < rem && rem <= incl) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (run + (int64_t)v[u] >= rem) {
                st->key_prefix = base | ((uint64_t)(4 * t + u) << lo);
                st->k_tie = rem - run;
                st->ksel_fix = lo;
                st->ksel_n = 0;
                st->ksel_state = lo == 0 ? 2 : 1;
                break;
            }
            run += v[u];
        }
    }
}

// The ties in the cut bucket (bits >= ksel_fix equal the prefix): counted,
// and gathered into sel while they fit.
__global__ __launch_bounds__(kThreads) void k_lru_bucket(LruState* __restrict__ st, const uint64_t* __restrict__ ties,
                                                        const int32_t* __restrict__ tie_cnt, int64_t nchunks,
                                                        uint64_t* __restrict__ sel, int use_log, int log_chunk) {
    if (st->k <= 0 || st->ksel_state != 1) return;
    const int64_t nb = busy_chunks(st, nchunks, use_log, log_chunk);
    const uint64_t want = st->key_prefix;
    const int fix = st->ksel_fix;
    const int lane = lane_id();
    for_wave_chunks(tie_cnt, nb, nullptr, [&](int64_t c, int cnt) {
        for (int j0 = 0; j0 < cnt; j0 += 64) {
            const int j = j0 + lane;
            uint64_t x = 0;
            bool in = false;
            if (j < cnt) {
                x = ties[c * kChunk + j];
                in = ksel_match(x, want, fix);
            }
            const uint64_t m = __ballot(in);
            if (m) {
                int at = 0;
                if (lane == 0) at = atomicAdd(&st->ksel_n, __popcll(m));
                at = __shfl(at, 0) + __popcll(m & lanemask_lt());
                if (in && at < kFinalCap) sel[at] = x;
            }
        }
    });
}

// Calls f(c, cnt) for every chunk c < n with a nonzero count, over the 16
// waves of a 1024-thread block, 64 counts loaded at once per wave.
template <class F>
__device__ __forceinline__ void for_block_chunks(const int32_t* __restrict__ cnts, int64_t n, F&& f) {
    const int lane = lane_id();
    for (int64_t c0 = (int64_t)(threadIdx.x >> 6) * 64; c0 < n; c0 += 1024) {
        const int64_t c = c0 + lane;
        const int32_t cnt = c < n ? cnts[c] : 0;
        uint64_t busy = __ballot(cnt > 0);
        while (busy) {
            const int j = __ffsll((long long)busy) - 1;
            busy &= busy - 1;
            f(c0 + j, __shfl(cnt, j));
        }
    }
}

// One block: the cut key among the bucket's ties.  Up to kFinalCap of them
// were gathered into sel: ranked in LDS (keys are distinct: exactly one has
// k_rem - 1 smaller ones).  More are narrowed by 8-bit radix passes over the
// bits below the window, each a pass over all the ties (those off the
// prefix are skipped).
__global__ __launch_bounds__(1024) void k_lru_final(LruState* __restrict__ st, const uint64_t* __restrict__ ties,
                                                   const int32_t* __restrict__ tie_cnt, int64_t nchunks,
                                                   const uint64_t* __restrict__ sel, int use_log, int log_chunk) {
    __shared__ uint64_t s_k[kFinalCap];
    __shared__ uint32_t s_h[256];
    __shared__ int64_t s_w[1024 / 64];
    __shared__ uint64_t s_prefix;
    __shared__ int64_t s_rem;
    if (st->k <= 0 || st->ksel_state != 1) return;
    const int t = threadIdx.x;
    const int m = st->ksel_n;
    if (m <= kFinalCap) {
        for (int i = t; i < m; i += 1024) s_k[i] = sel[i];
        __syncthreads();
        const int64_t rem = st->k_tie;
        for (int i = t; i < m; i += 1024) {
            const uint64_t x = s_k[i];
            int below = 0;
            for (int j = 0; j < m; ++j) below += s_k[j] < x ? 1 : 0;
            if (below == rem - 1) st->key_prefix = x;
        }
        if (t == 0) st->ksel_state = 2;
        return;
    }
    const int64_t nb = busy_chunks(st, nchunks, use_log, log_chunk);
    if (t == 0) {
        s_prefix = st->key_prefix;
        s_rem = st->k_tie;
    }
    int fix = st->ksel_fix;
    __syncthreads();
    while (fix > 0) {
        const int lo = fix > 8 ? fix - 8 : 0;
        const uint32_t mask = (1u << (fix - lo)) - 1u;
        const uint64_t want = s_prefix;
        if (t < 256) s_h[t] = 0u;
        __syncthreads();
        const int lane = lane_id();
        for_block_chunks(tie_cnt, nb, [&](int64_t c, int cnt) {
            for (int j = lane; j < cnt; j += 64) {
                const uint64_t x = ties[c * kChunk + j];
                if (ksel_match(x, want, fix)) atomicAdd(&s_h[(uint32_t)(x >> lo) & mask], 1u);
            }
        });
        __syncthreads();
        const int64_t h = t < 256 ? (int64_t)s_h[t] : 0;
        const int64_t incl = scan1024(h, s_w);
        const int64_t rem = s_rem;
        __syncthreads();
        if (t < 256 && incl - h < rem && rem <= incl) {
            s_prefix = want | ((uint64_t)t << lo);
            s_rem = rem - (incl - h);
        }
        __syncthreads();
        fix = lo;
    }
    if (t == 0) {
        st->key_prefix = s_prefix;
        st->k_tie = s_rem;
        st->ksel_state = 2;
    }
}

// One block: exclusive prefix of the per-chunk victim counts, in rounds of
// 4096 chunks (four per thread, loaded as one 16-byte vector), carrying the
// running total; with the access log only the window's chunks (the others
// hold no candidate and their offsets are not read).
__global__ __launch_bounds__(1024) void k_lru_offsets(const LruState* __restrict__ st, const int32_t* __restrict__ cnt,
                                                     int64_t nchunks, int32_t* __restrict__ off, int use_log,
                                                     int log_chunk) {
    __shared__ int64_t s_w[1024 / 64];
    __shared__ int64_t s_carry;
    const int64_t nb = busy_chunks(st, nchunks, use_log, log_chunk);
    const int t = threadIdx.x;
    if (t == 0) s_carry = 0;
    for (int64_t c0 = 0; c0 < nb; c0 += 4096) {
        const int64_t c = c0 + 4 * t;
        int32_t v[4];
        if (c + 3 < nchunks && (nchunks & 3) == 0) {
            const int4 x = *reinterpret_cast<const int4*>(cnt + c);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = c + u < nchunks ? cnt[c + u] : 0;
        }
        const int64_t sum = (int64_t)v[0] + v[1] + v[2] + v[3];
        const int64_t incl = scan1024(sum, s_w);      // its barriers also order s_carry
        int64_t run = s_carry + incl - sum;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (c + u < nchunks) off[c + u] = (int32_t)run;
            run += v[u];
        }
        __syncthreads();
        if (t == 1023) s_carry = run;
        __syncthreads();
    }
}

// A chunk's victims: its candidates below the cut last_seen, then its ties
// at or below the cut key -- taken from the ties array, which holds their
// keys, so that keys are read through the slot only for the victims below
// the cut.  The victim passes take one chunk per wave (c = w + i * W over
// the grid's waves), with wave-wide prefixes.
__global__ __launch_bounds__(kThreads) void k_lru_count_victims(const LruState* __restrict__ st,
                                                               const uint32_t* __restrict__ cand_ls,
                                                               const int32_t* __restrict__ chunk_cnt,
                                                               const uint64_t* __restrict__ ties,
                                                               const int32_t* __restrict__ tie_cnt,
                                                               int64_t nchunks, int32_t* __restrict__ vic_cnt,
                                                               int use_log, int log_chunk) {
    const bool any = st->k > 0;
    const uint32_t thr = st->ls_cut;
    const uint64_t kthr = st->key_prefix;
    const int lane = lane_id();
    nchunks = busy_chunks(st, nchunks, use_log, log_chunk);
    const int64_t W = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t c = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); c < nchunks; c += W) {
        const int cnt = any ? chunk_cnt[c] : 0;
        const int tc = any ? tie_cnt[c] : 0;
        int tot = 0;
        for (int j0 = 0; j0 < cnt; j0 += 64) {
            const int j = j0 + lane;
            tot += __popcll(__ballot(j < cnt && cand_ls[c * kChunk + j] < thr));
        }
        for (int j0 = 0; j0 < tc; j0 += 64) {
            const int j = j0 + lane;
            tot += __popcll(__ballot(j < tc && ties[c * kChunk + j] <= kthr));
        }
        if (lane == 0) vic_cnt[c] = tot;
    }
}

__global__ __launch_bounds__(kThreads) void k_lru_emit(const LruState* __restrict__ st,
                                                      const uint32_t* __restrict__ cand_ls,
                                                      const uint32_t* __restrict__ cand_slot,
                                                      const int64_t* __restrict__ keys,
                                                      const int32_t* __restrict__ chunk_cnt,
                                                      const uint64_t* __restrict__ ties,
                                                      const int32_t* __restrict__ tie_cnt, int64_t nchunks,
                                                      const int32_t* __restrict__ vic_off, int64_t* __restrict__ victims,
                                                      int64_t cap, int64_t* __restrict__ n_victims, int use_log,
                                                      int log_chunk) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_victims = st->k;
    const bool any = st->k > 0;
    const uint32_t thr = st->ls_cut;
    const uint64_t kthr = st->key_prefix;
    const int lane = lane_id();
    nchunks = busy_chunks(st, nchunks, use_log, log_chunk);
    const int64_t W = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t c = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); c < nchunks; c += W) {
        const int cnt = any ? chunk_cnt[c] : 0;
        const int tc = any ? tie_cnt[c] : 0;
        int64_t run = vic_off[c];
        for (int j0 = 0; j0 < cnt; j0 += 64) {
            const int j = j0 + lane;
            const bool v = j < cnt && cand_ls[c * kChunk + j] < thr;
            int64_t key = 0;
            if (v) key = keys[cand_slot[c * kChunk + j]];
            const uint64_t m = __ballot(v);
            const int64_t at = run + __popcll(m & lanemask_lt());
            if (v && at < cap) victims[at] = key;
            run += __popcll(m);
        }
        for (int j0 = 0; j0 < tc; j0 += 64) {
            const int j = j0 + lane;
            uint64_t x = 0;
            if (j < tc) x = ties[c * kChunk + j];
            const bool v = j < tc && x <= kthr;
            const uint64_t m = __ballot(v);
            const int64_t at = run + __popcll(m & lanemask_lt());
            if (v && at < cap) victims[at] = (int64_t)bias((int64_t)x);   // unbias: the flip is its own inverse
            run += __popcll(m);
        }
    }
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

size_t lru_workspace_bytes(const htl_table* t) {
    if (!t) return 0;
    return lru_layout(t->dev.capacity, nullptr).bytes;
}

htl_status ht_lru_select(const htl_table* t, int64_t num, int64_t den, int64_t* victims, int64_t victims_cap,
                         int64_t* n_victims_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_lru_select: null table");
    HTL_REQUIRE(t->dev.last_seen != nullptr, "ht_lru_select: table keeps no last_seen (HT_META_LAST_SEEN)");
    HTL_REQUIRE(den >= 1 && den <= ((int64_t)1 << 31) && num >= 0 && num <= den,
                "ht_lru_select: need 0 <= num <= den <= 2^31");
    HTL_REQUIRE(victims_cap >= 0, "ht_lru_select: negative victims_cap");
    HTL_REQUIRE(n_victims_dev && aligned(n_victims_dev, 8) && ws && aligned(ws, 256) &&
                    (victims_cap == 0 || (victims && aligned(victims, 8))),
                "ht_lru_select: null or misaligned pointer");
    HTL_REQUIRE(t->capacity_log2 <= 30, "ht_lru_select: needs capacity_log2 <= 30");
    LruWs w = lru_layout(t->dev.capacity, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "ht_lru_select: workspace too small");
    const TableDev& T = t->dev;
    const unsigned gchunk = grid_for(w.nchunks, 1, 1 << 16);
    const unsigned gwave = grid_for(w.nchunks, kThreads / 64, 1 << 16);   // a chunk per wave
    const unsigned ghist = grid_for(w.nchunks, 1, kHistBlocks);
    // with an access log that serves, the cut step comes from its step counts
    // and the candidates from its ring (the log's own kernel decides on the
    // device whether it serves: the kernels below follow its choice)
    const int use_log = (t->log.entries && t->log_ok) ? 1 : 0;
    if (use_log)
        hipLaunchKernelGGL(k_lru_log_init, dim3(1), dim3(1024), 0, stream, w.st, t->log, t->log_par, t->max_step, num,
                           den);
    int log_chunk = kChunk;
    if (use_log) {
        const int64_t per = (int64_t)(t->log.cap_mask + 1) / w.nchunks;
        log_chunk = per < kChunk ? (int)per : kChunk;
    }
    hipLaunchKernelGGL(k_lru_collect, dim3(gchunk), dim3(kThreads), 0, stream, T, w.nchunks, w.cand_ls, w.cand_slot,
                       w.chunk_cnt, w.chunk_max, use_log, t->log, (const LruState*)w.st, log_chunk);
    hipLaunchKernelGGL(k_lru_init, dim3(1), dim3(1024), 0, stream, w.st, w.chunk_cnt, w.chunk_max, w.nchunks, num,
                       den, use_log);
    // last_seen digits: as many as the largest step stamped needs (the
    // kernels also skip digits above the live maximum)
    int ls_digits = 1;
    while (ls_digits < 4 && (t->max_step >> (8 * ls_digits)) != 0u) ++ls_digits;
    for (int d = ls_digits - 1; d >= 0; --d) {
        hipLaunchKernelGGL(k_lru_hist_ls, dim3(ghist), dim3(kThreads), 0, stream, w.st, w.cand_ls, w.chunk_cnt,
                           w.nchunks, d);
        // the last digit's pick runs inside k_lru_ties
        if (d > 0) hipLaunchKernelGGL(k_lru_pick, dim3(1), dim3(256), 0, stream, w.st, d);
    }
    hipLaunchKernelGGL(k_lru_ties, dim3(ghist), dim3(kThreads), 0, stream, w.st, w.cand_ls, w.cand_slot, T.keys,
                       w.chunk_cnt, w.nchunks, w.ties, w.tie_cnt, w.khist, use_log, log_chunk);
    hipLaunchKernelGGL(k_lru_hist_key, dim3(ghist), dim3(kThreads), 0, stream, (const LruState*)w.st, w.ties,
                       w.tie_cnt, w.nchunks, w.khist, use_log, log_chunk);
    hipLaunchKernelGGL(k_lru_pick_key, dim3(1), dim3(1024), 0, stream, w.st, w.khist);
    hipLaunchKernelGGL(k_lru_bucket, dim3(ghist), dim3(kThreads), 0, stream, w.st, w.ties, w.tie_cnt, w.nchunks,
                       w.sel, use_log, log_chunk);
    hipLaunchKernelGGL(k_lru_final, dim3(1), dim3(1024), 0, stream, w.st, w.ties, w.tie_cnt, w.nchunks, w.sel,
                       use_log, log_chunk);
    hipLaunchKernelGGL(k_lru_count_victims, dim3(gwave), dim3(kThreads), 0, stream, w.st, w.cand_ls, w.chunk_cnt,
                       w.ties, w.tie_cnt, w.nchunks, w.vic_cnt, use_log, log_chunk);
    hipLaunchKernelGGL(k_lru_offsets, dim3(1), dim3(1024), 0, stream, (const LruState*)w.st, w.vic_cnt, w.nchunks,
                       w.vic_off, use_log, log_chunk);
    hipLaunchKernelGGL(k_lru_emit, dim3(gwave), dim3(kThreads), 0, stream, w.st, w.cand_ls, w.cand_slot, T.keys,
                       w.chunk_cnt, w.ties, w.tie_cnt, w.nchunks, w.vic_off, victims, victims_cap, n_victims_dev,
                       use_log, log_chunk);
    return check_launch("ht_lru_select");
}

}  // extern "C"
