// Two-stage feature-ID deduplication: unique keys plus inverse index.
//
// MTGenRec (arXiv 2505.12663), TL;DR and section 6 of its contents ("Embedding
// Table Lookup Acceleration"): the IDs are deduplicated in two stages so
// that the embedding lookup is quicker.  MTGR (arXiv 2505.18654) section 5,
// "Embedding Lookup":
// IDs are made unique before and after the cross-device all-to-all so that no
// duplicate crosses the link.  On one device the two stages become:
//
//   stage 1 (k_dedup_tile): each workgroup dedups one tile of kTile keys in an
//     LDS open-addressing set (2*kTile slots, 64-bit ds CAS), writes the tile's
//     distinct keys compactly to its own region in order of first occurrence,
//     and a 16-bit local index per key.  One copy of each key leaves the tile,
//     as one copy per sender would leave a device before the exchange; under
//     Zipf traffic this also turns the hottest key's thousands of global
//     atomics into at most one per tile.  The same grid first clears the
//     stage-2 set (no launch of its own; its stores stream out while the
//     tiles work in LDS).
//   stage 2 (k_dedup_claim, [k_dedup_count], k_dedup_assign): every tile
//     survivor is inserted into a device-wide open-addressing set
//     (next_pow2(3n/2 + 1) slots, 64-bit CAS).  One survivor per key owns
//     it: the one whose CAS inserted it, or, in ordered mode, the one in the lowest
//     tile (atomicMin).  Per-tile counts of owned keys are prefix-summed and
//     owned keys take dense ids in tile order -- no counter atomics.  In
//     ordered mode the ids, hence `unique`, follow the order of first
//     occurrence in the batch; that costs one more atomic per unique key and
//     two more random reads per survivor.
//   compose (k_dedup_compose): inverse[i] = id(set slot of tile survivor
//     local[i]), one workgroup per tile with the survivors' ids in LDS.
//
// Stage 2 has a second form, hash-partitioned, that needs no global atomics
// (a device-scope CAS costs as much as three or four random loads on this
// part, whatever the working set):
//   k_part_count counts the survivors of each row of tiles per hash bin (P
//     bins, the top bits of a salted mix);
//   k_col_scan turns the row x bin counts into the place of each (row, bin)
//     run inside its bin and the bins' totals; the bins' bases in the
//     bin-major survivor array are the prefix of the totals;
//   k_part_scatter moves every survivor (key, tile position) there; rows are
//     spread over the XCDs in contiguous runs, so each XCD writes contiguous
//     pieces of every bin and its L2 merges them into whole lines;
//   k_part_dedup: one workgroup per bin dedups the bin's survivors in an LDS
//     set (ids in order of arrival: per round of survivors, the inserting
//     ones in thread order), writes the bin's distinct keys and, at each
//     survivor's tile position, its id inside the bin; a bin with more
//     distinct keys than its LDS set holds is redone in a region of device
//     memory of its own;
//   k_part_finish: the bins' distinct keys are packed by the prefix of their
//     counts (unique = bin-major), and the inverse is composed per tile from
//     (bin offset + id in bin) -- no random reads.
//
// Adaptive choice (the TensorFlow article, section 3.6: a heuristic picks the
// Unique implementation): a batch of at most one tile (2048 keys, e.g. a
// serving request) is deduplicated by the LDS stage alone in one launch; the
// device set and its clear, the claim, the scan and the compose are skipped.
// Larger batches of up to 2^23 keys take the partitioned stage 2 in the
// unordered mode; the ordered mode, and larger batches, take the set (above
// 2^23 keys each row's run per bin shrinks below a cache line and the
// scatter falls behind).
//
// The LDS sets and the device set probe with an odd step over a power-of-two
// capacity, so by MTGenRec's Theorem 1 a probe walk reaches every slot; with
// at most n keys in more than 3n/2 slots the device set's walk always ends
// at a free slot (load at most 2/3: the set is cleared on every call, so its
// size is traded against that clear).  A bin redone in device memory walks
// with step 1 over 2*cnt + 1 slots, so it too reaches every slot and never
// fills.
// The set is capped at 2^30 slots (its slot numbers, and the extra entry of
// key -1 at index 2^30, stay int32); with n < 2^30 a slot is always free.
// Every int64 is a valid key: the value -1, which both sets use as their
// empty marker, is carried out of band.
#include <atomic>
#include <cstring>
#include <new>

#include "debug.h"
#include "lookup.h"
#include "scan.h"
#include "tile_dedup.h"

namespace htl {
namespace {

struct DedupWs {
    unsigned long long* set_keys;   // [cap]
    int32_t* set_owner;             // [cap + 1]: lowest tile holding the key (entry cap: key -1)
    int32_t* set_ids;               // [cap + 1]: dense id of the key
    int64_t* tu_keys;               // [ntiles * kTile]: per-tile distinct keys, first-occurrence order
    int32_t* tu_slot;               // [ntiles * kTile]: their set slot (cap: key -1)
    uint8_t* tu_own;                // [ntiles * kTile]: 1 if this survivor owns its key
    int32_t* tu_count;              // [ntiles]
    int32_t* misc;                  // [0]: key -1 claimed (unordered mode)
    int32_t* tile_win;              // [ntiles]: keys each tile owns
    int32_t* tile_off;              // [ntiles + 1]: exclusive prefix of tile_win
    void* scan_tmp;
    uint16_t* local;                // [n]
    uint64_t cap;
    size_t bytes;
};

DedupWs layout(int64_t n, char* base) {
    DedupWs w{};
    const int64_t ntiles = ceil_div(n, kTile);
    uint64_t cap = 256;
    while (cap <= (uint64_t)(n + n / 2) && cap < ((uint64_t)1 << 30)) cap <<= 1;   // slot indices stay int32
    w.cap = cap;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.set_keys = (unsigned long long*)take(cap * 8);
    w.set_owner = (int32_t*)take((cap + 1) * 4);
    w.set_ids = (int32_t*)take((cap + 1) * 4);
    w.tu_keys = (int64_t*)take((size_t)ntiles * kTile * 8);
    w.tu_slot = (int32_t*)take((size_t)ntiles * kTile * 4);
    w.tu_own = (uint8_t*)take((size_t)ntiles * kTile);
    w.tu_count = (int32_t*)take((size_t)ntiles * 4);
    w.misc = (int32_t*)take(256);
    w.tile_win = (int32_t*)take((size_t)ntiles * 4);
    w.tile_off = (int32_t*)take((size_t)(ntiles + 1) * 4);
    w.scan_tmp = take(scan_temp_bytes(ntiles));
    w.local = (uint16_t*)take((size_t)n * 2);
    w.bytes = off;
    return w;
}

constexpr int kGlobalThreads = kTileThreads;

// Stage 2a: every tile survivor is put in the device-wide set.  A slot is
// read before any atomic: a key already in the set (the usual case for
// Zipf-hot keys, which every tile carries) costs a cacheable load, not an
// atomic that would serialise with the same key's atomics from every other
// tile.  A CAS is attempted only on a slot seen EMPTY; if it loses, the value
// it returns decides (same key: found; other key: walk on).
// Ownership: unordered mode -- the survivor whose CAS inserted the key owns
// it, and the block counts its tile's owners right here; ordered mode -- the
// lowest tile holding the key owns it (atomicMin on the slot's owner field,
// again read first), counted by k_dedup_count once every tile is done.
template <bool ORDERED>
__global__ __launch_bounds__(kGlobalThreads) void k_dedup_claim(
    const int64_t* __restrict__ tu_keys, const int32_t* __restrict__ tu_count, int64_t ntiles,
    unsigned long long* __restrict__ set_keys, int32_t* __restrict__ set_owner, uint64_t set_mask,
    int32_t* __restrict__ tu_slot, uint8_t* __restrict__ tu_own, int32_t* __restrict__ tile_win,
    int32_t* __restrict__ misc) {
    __shared__ int s_wave[kGlobalThreads / 64];
    const uint64_t cap = set_mask + 1;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        int owned = 0;
        for (int j = threadIdx.x; j < cnt; j += kGlobalThreads) {
            const uint64_t k = (uint64_t)tu_keys[tile * kTile + j];
            uint64_t p = cap;                        // key -1: the extra entry
            bool won = false;
            if (k != kFree) {
                const uint64_t h = mix64(k ^ kSalt2);
                p = h & set_mask;
                const uint64_t stp = ((h >> 32) | 1ull) & set_mask;
                for (uint64_t probe = 0; probe <= set_mask; ++probe) {
                    const uint64_t cur = peek_u64(&set_keys[p]);
                    if (cur == k) break;
                    if (cur == kFree) {
                        const unsigned long long old = atomicCAS(&set_keys[p], kFree, (unsigned long long)k);
                        if (old == kFree) {
                            won = true;
                            break;
                        }
                        if (old == k) break;
                    }
                    p = (p + stp) & set_mask;
                }
            } else if (!ORDERED) {
                if (__hip_atomic_load(&misc[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
                    won = atomicCAS(&misc[0], 0, 1) == 0;
            }
            if (ORDERED) {
                const int32_t t32 = (int32_t)tile;
                if (__hip_atomic_load(&set_owner[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > t32)
                    atomicMin(&set_owner[p], t32);
            } else {
                tu_own[tile * kTile + j] = won ? 1 : 0;
                owned += won;
            }
            tu_slot[tile * kTile + j] = (int32_t)p;
        }
        if (!ORDERED) {
            for (int off = 32; off > 0; off >>= 1) owned += __shfl_xor(owned, off);
            if (lane_id() == 0) s_wave[threadIdx.x >> 6] = owned;
            __syncthreads();
            if (threadIdx.x == 0) {
                int tot = 0;
                for (int w = 0; w < kGlobalThreads / 64; ++w) tot += s_wave[w];
                tile_win[tile] = tot;
            }
            __syncthreads();
        }
    }
}

// Stage 2b (ordered mode): how many of its keys each tile owns.
__global__ __launch_bounds__(kGlobalThreads) void k_dedup_count(const int32_t* __restrict__ tu_count,
                                                               const int32_t* __restrict__ tu_slot, int64_t ntiles,
                                                               const int32_t* __restrict__ set_owner,
                                                               int32_t* __restrict__ tile_win) {
    __shared__ int s_wave[kGlobalThreads / 64];
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        int mine = 0;
        for (int j = threadIdx.x; j < cnt; j += kGlobalThreads)
            mine += set_owner[tu_slot[tile * kTile + j]] == (int32_t)tile;
        for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off);
        if (lane_id() == 0) s_wave[threadIdx.x >> 6] = mine;
        __syncthreads();
        if (threadIdx.x == 0) {
            int tot = 0;
            for (int w = 0; w < kGlobalThreads / 64; ++w) tot += s_wave[w];
            tile_win[tile] = tot;
        }
        __syncthreads();
    }
}

// Stage 2c: owned keys get dense ids in (tile, position in tile) order.  In
// ordered mode that is the order of first occurrence in the whole batch.
// An owner also leaves its id in its own survivor entry (tu_slot becomes
// -(id + 1)), so that compose reads it there, in sequence, and only the
// survivors that do not own their key read the id at the set slot.
template <bool ORDERED>
__global__ __launch_bounds__(kGlobalThreads) void k_dedup_assign(
    const int64_t* __restrict__ tu_keys, const int32_t* __restrict__ tu_count, int32_t* __restrict__ tu_slot,
    const uint8_t* __restrict__ tu_own, int64_t ntiles, const int32_t* __restrict__ set_owner,
    const int32_t* __restrict__ tile_off, int32_t* __restrict__ set_ids, int64_t* __restrict__ unique,
    int64_t* __restrict__ n_unique) {
    __shared__ int s_wave[kGlobalThreads / 64];
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_unique = tile_off[ntiles];
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        int run = tile_off[tile];
        for (int jb = 0; jb < cnt; jb += kGlobalThreads) {
            const int j = jb + threadIdx.x;
            int32_t p = 0;
            bool own = false;
            if (j < cnt) {
                p = tu_slot[tile * kTile + j];
                own = ORDERED ? set_owner[p] == (int32_t)tile : tu_own[tile * kTile + j] != 0;
            }
            int tot;
            const int r = block_rank(own, s_wave, &tot);
            if (own) {
                set_ids[p] = run + r;
                unique[run + r] = tu_keys[tile * kTile + j];
                tu_slot[tile * kTile + j] = -(run + r) - 1;
            }
            run += tot;
        }
    }
}

// inverse[i] = id of the set slot of tile survivor local[i]: each block takes
// one tile, fetches its survivors' ids once into LDS (an owner's from its
// own entry, the others' from the set), then maps its IDs.  With `slots`
// (the find-or-insert result of `unique`), each survivor also fetches its
// key's slot once, and sid[i] = slots[inverse[i]] is written beside the
// inverse, so that a later gather reads one index per ID, in sequence.
__global__ __launch_bounds__(kTileThreads) void k_dedup_compose(const uint16_t* __restrict__ local, int64_t n,
                                                               const int32_t* __restrict__ tu_count,
                                                               const int32_t* __restrict__ tu_slot,
                                                               const int32_t* __restrict__ set_ids,
                                                               int32_t* __restrict__ inverse,
                                                               const int32_t* __restrict__ slots,
                                                               int32_t* __restrict__ sid) {
    __shared__ int32_t s_gid[kTile];
    __shared__ int32_t s_sl[kTile];
    for (int64_t tile = blockIdx.x; tile * kTile < n; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        // each hop's loads for all of a thread's survivors are issued together
        // (merged-tables step 2.666 -> 2.652 ms against one survivor at a time)
        constexpr int kPer = kTile / kTileThreads;
        int32_t v[kPer], g[kPer], sl[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int j = k * kTileThreads + threadIdx.x;
            v[k] = j < cnt ? tu_slot[tile * kTile + j] : -1;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) g[k] = v[k] < 0 ? -(v[k] + 1) : set_ids[v[k]];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int j = k * kTileThreads + threadIdx.x;
            sl[k] = (slots && j < cnt) ? slots[g[k]] : 0;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int j = k * kTileThreads + threadIdx.x;
            if (j < cnt) {
                s_gid[j] = g[k];
                if (slots) s_sl[j] = sl[k];
            }
        }
        __syncthreads();
        const int64_t base = tile * kTile;
        for (int q = threadIdx.x; q < kTile; q += kTileThreads) {
            const int64_t i = base + q;
            if (i < n) {
                const int l = local[i];
                inverse[i] = s_gid[l];
                if (slots) sid[i] = s_sl[l];
            }
        }
        __syncthreads();
    }
}

__global__ void k_write_zero(int64_t* p) { *p = 0; }

// Stage 2 without stage 1: every tile's "survivors" are its keys, as many
// as the tile holds.
__global__ void k_tile_lengths(int32_t* __restrict__ tu_count, int64_t n, int64_t ntiles) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < ntiles; t += (int64_t)gridDim.x * blockDim.x)
        tu_count[t] = (int32_t)(n - t * kTile < kTile ? n - t * kTile : kTile);
}

// ------------------------------------------------ partitioned stage 2 ----
constexpr int kPartMinLog2 = 8;               // bins: 2^8 .. 2^12
constexpr int kPartMaxLog2 = 12;
constexpr int kPartRowsMax = 1024;            // rows of tiles (count-matrix height)
constexpr int kColChunk = 32;                 // rows per partial column sum
constexpr int kChunksMax = kPartRowsMax / kColChunk;   // 32
constexpr int64_t kPartMaxN = (int64_t)1 << 23;   // larger batches: the device set (see run_dedup)
constexpr int kRowThreads = 1024;             // count and scatter passes
constexpr int kRowVec = 4;                    // survivor slots per thread in flight
constexpr int kBinThreads = 512;
constexpr int kBinVec = 4;                    // survivors per thread per round of a bin
constexpr int kBinSet = 4096;                 // LDS set slots of one bin
constexpr int kBinMax = kBinSet * 7 / 10;     // distinct keys a bin may hold in LDS

struct PartWs {
    int64_t* tu_keys;      // [ntiles * kTile]: per-tile distinct keys
    int32_t* tu_count;     // [ntiles]
    int32_t* tu_l;         // [ntiles * kTile]: id of the survivor's key inside its bin
    uint16_t* local;       // [n]
    int32_t* cnt;          // [rows << plog2]: counts, then run offsets
    int32_t* btotal;       // [bins]: survivors per bin
    int32_t* base;         // [bins + 1]: start of each bin in the bin-major array
    u32x4* ent;            // [n]: bin-major survivors (key lo, key hi, tile slot, 0)
    int64_t* ustage;       // [n]: each bin's distinct keys at the bin's start
    int32_t* ucount;       // [bins]
    int32_t* uoff;         // [bins + 1]: exclusive prefix of ucount
    unsigned long long* fb_keys;   // [2n + bins]: sets of bins past the LDS set
    int32_t* fb_ids;       // [2n + bins]
    int plog2, rows, tpr;
    size_t bytes;
};

PartWs part_layout(int64_t n, char* base) {
    PartWs w{};
    const int64_t ntiles = ceil_div(n, kTile);
    int plog2 = kPartMinLog2;
    while (plog2 < kPartMaxLog2 && ((int64_t)1 << plog2) < ntiles) ++plog2;
    const int64_t P = (int64_t)1 << plog2;
    w.plog2 = plog2;
    w.tpr = (int)ceil_div(ntiles, kPartRowsMax);
    w.rows = (int)ceil_div(ntiles, w.tpr);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.tu_keys = (int64_t*)take((size_t)ntiles * kTile * 8);
    w.tu_count = (int32_t*)take((size_t)ntiles * 4);
    w.tu_l = (int32_t*)take((size_t)ntiles * kTile * 4);
    w.local = (uint16_t*)take((size_t)n * 2);
    w.cnt = (int32_t*)take((size_t)w.rows * P * 4);
    w.btotal = (int32_t*)take((size_t)P * 4);
    w.base = (int32_t*)take((size_t)(P + 1) * 4);
    w.ent = (u32x4*)take((size_t)n * 16);
    w.ustage = (int64_t*)take((size_t)n * 8);
    w.ucount = (int32_t*)take((size_t)P * 4);
    w.uoff = (int32_t*)take((size_t)(P + 1) * 4);
    w.fb_keys = (unsigned long long*)take((size_t)(2 * n + P) * 8);
    w.fb_ids = (int32_t*)take((size_t)(2 * n + P) * 4);
    w.bytes = off;
    return w;
}

// Row of the count matrix that block `bid` of a rows-wide grid takes: the
// rows are dealt to the 8 XCDs (workgroups go round-robin over them) in
// contiguous runs, so one XCD's concurrent rows write adjacent pieces of
// each bin.  A bijection of [0, rows) onto itself.
__device__ __forceinline__ int xcd_row(int bid, int rows) {
    const int q = rows >> 3, rem = rows & 7;
    const int x = bid & 7, i = bid >> 3;
    return x < rem ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
}

// The survivor slots of row r are [t0 * kTile, t1 * kTile) of the tile-major
// arrays; slot s holds a survivor iff s mod kTile < tu_count[s / kTile].
// Loads kRowVec slots per thread at once; returns a bit per live slot.
__device__ __forceinline__ uint32_t load_row_slots(const int64_t* __restrict__ tu_keys,
                                                   const int32_t* __restrict__ tu_count, int64_t s0, int64_t s1,
                                                   uint64_t* k, int64_t* slot) {
    uint32_t live = 0;
#pragma unroll
    for (int u = 0; u < kRowVec; ++u) {
        const int64_t s = s0 + u * kRowThreads + threadIdx.x;
        slot[u] = s;
        k[u] = 0;
        if (s < s1 && (int)(s & (kTile - 1)) < tu_count[s >> kTileLog2]) {
            k[u] = (uint64_t)tu_keys[s];
            live |= 1u << u;
        }
    }
    return live;
}

// cnt[r][b] = survivors of row r's tiles in bin b.
__global__ __launch_bounds__(kRowThreads) void k_part_count(const int64_t* __restrict__ tu_keys,
                                                           const int32_t* __restrict__ tu_count, int64_t ntiles,
                                                           int tpr, int plog2, int32_t* __restrict__ cnt) {
    extern __shared__ int32_t s_hist[];   // [1 << plog2]
    const int r = blockIdx.x;
    for (int b = threadIdx.x; b < (1 << plog2); b += kRowThreads) s_hist[b] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)r * tpr;
    const int64_t t1 = t0 + tpr < ntiles ? t0 + tpr : ntiles;
    for (int64_t s0 = t0 * kTile; s0 < t1 * kTile; s0 += kRowThreads * kRowVec) {
        uint64_t k[kRowVec];
        int64_t slot[kRowVec];
        const uint32_t live = load_row_slots(tu_keys, tu_count, s0, t1 * kTile, k, slot);
#pragma unroll
        for (int u = 0; u < kRowVec; ++u)
            if (live & (1u << u)) atomicAdd(&s_hist[part_bin(k[u], plog2)], 1);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < (1 << plog2); b += kRowThreads) cnt[((int64_t)r << plog2) + b] = s_hist[b];
}

// The column pass over the row-major count matrix.  A workgroup takes 32
// bins and every chunk of kColChunk rows (thread = (chunk, bin)): it sums
// each chunk's rows, takes per bin the prefix of the chunk sums in LDS, and
// rewrites cnt[r][b] in place as the rows of bin b before row r; total[b] =
// all rows of bin b.  The bins' own bases (prefix of total) are taken by the
// kernels that need them.
constexpr int kColBins = 1024 / kChunksMax;            // bins per workgroup

__global__ __launch_bounds__(1024) void k_col_scan(int32_t* __restrict__ cnt, int rows, int plog2,
                                                  int32_t* __restrict__ total) {
    __shared__ int32_t s_c[kChunksMax][kColBins];
    const int bl = threadIdx.x % kColBins;
    const int c = threadIdx.x / kColBins;
    const int b = blockIdx.x * kColBins + bl;
    const int r0 = c * kColChunk;
    int32_t v[kColChunk];
#pragma unroll
    for (int j = 0; j < kColChunk; ++j) v[j] = r0 + j < rows ? cnt[((int64_t)(r0 + j) << plog2) + b] : 0;
    int32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kColChunk; ++j) sum += v[j];
    s_c[c][bl] = sum;
    __syncthreads();
    int32_t run = 0, all = 0;
#pragma unroll
    for (int c2 = 0; c2 < kChunksMax; ++c2) {
        const int32_t x = s_c[c2][bl];
        run += c2 < c ? x : 0;
        all += x;
    }
#pragma unroll
    for (int j = 0; j < kColChunk; ++j) {
        if (r0 + j < rows) cnt[((int64_t)(r0 + j) << plog2) + b] = run;
        run += v[j];
    }
    if (c == 0) total[b] = all;
}

// Exclusive prefix of the P <= 4096 bin totals in LDS by one workgroup of
// kRowThreads threads (4 bins per thread); s_w holds kRowThreads / 64 ints.
__device__ __forceinline__ void bin_bases(const int32_t* __restrict__ total, int P, int32_t* s_base, int* s_w) {
    int t[4];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = threadIdx.x * 4 + u;
        t[u] = b < P ? total[b] : 0;
        sum += t[u];
    }
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_w[wid] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wid; ++w) before += s_w[w];
    int run = before + incl - sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = threadIdx.x * 4 + u;
        if (b < P) s_base[b] = run;
        run += t[u];
    }
    __syncthreads();
}

constexpr int kBaseThreads = 1024;

// One workgroup: out[b] = sum of in[b'] for b' < b, out[P] = total (P <= 4096).
__global__ __launch_bounds__(kBaseThreads) void k_prefix_bins(const int32_t* __restrict__ in, int P,
                                                             int32_t* __restrict__ out) {
    __shared__ int s_w[kBaseThreads / 64];
    int t[4];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = threadIdx.x * 4 + u;
        t[u] = b < P ? in[b] : 0;
        sum += t[u];
    }
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_w[wid] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kBaseThreads / 64; ++w) {
        before += (w < wid) ? s_w[w] : 0;
        tot += s_w[w];
    }
    int run = before + incl - sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = threadIdx.x * 4 + u;
        if (b < P) out[b] = run;
        run += t[u];
    }
    if (threadIdx.x == 0) out[P] = tot;
}

// Every survivor of a row's tiles goes to its bin's run: (key, tile slot).
__global__ __launch_bounds__(kRowThreads) void k_part_scatter(const int64_t* __restrict__ tu_keys,
                                                             const int32_t* __restrict__ tu_count, int64_t ntiles,
                                                             const int32_t* __restrict__ cnt,
                                                             const int32_t* __restrict__ total, int rows, int tpr,
                                                             int plog2, u32x4* __restrict__ ent) {
    extern __shared__ int32_t s_cur[];   // [1 << plog2]
    __shared__ int s_w[kRowThreads / 64];
    const int r = xcd_row(blockIdx.x, rows);
    static_assert((1 << kPartMaxLog2) <= 4 * kRowThreads, "four bins per thread");
    bin_bases(total, 1 << plog2, s_cur, s_w);
    for (int b = threadIdx.x; b < (1 << plog2); b += kRowThreads) s_cur[b] += cnt[((int64_t)r << plog2) + b];
    __syncthreads();
    const int64_t t0 = (int64_t)r * tpr;
    const int64_t t1 = t0 + tpr < ntiles ? t0 + tpr : ntiles;
    for (int64_t s0 = t0 * kTile; s0 < t1 * kTile; s0 += kRowThreads * kRowVec) {
        uint64_t k[kRowVec];
        int64_t slot[kRowVec];
        const uint32_t live = load_row_slots(tu_keys, tu_count, s0, t1 * kTile, k, slot);
#pragma unroll
        for (int u = 0; u < kRowVec; ++u) {
            if (!(live & (1u << u))) continue;
            const int pos = atomicAdd(&s_cur[part_bin(k[u], plog2)], 1);
            u32x4 e;
            e.x = (uint32_t)k[u];
            e.y = (uint32_t)(k[u] >> 32);
            e.z = (uint32_t)slot[u];
            e.w = 0u;
            ent[pos] = e;
        }
    }
}

// Block-wide exclusive scan of one small count per thread (kBinThreads
// threads); returns the block total.  Uses s_wave[kBinThreads / 64].
__device__ __forceinline__ int bin_block_scan(int v, int* s_wave, int* total) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave[wid] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kBinThreads / 64; ++w) {
        const int c = s_wave[w];
        before += (w < wid) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return before + incl - v;
}

// One pass of a bin's dedup over its survivors ent[start, start + cnt), in
// rounds of kBinVec survivors per thread, into a set of `size` slots: LDS
// (GLOBAL false; size a power of two, odd-step walk) or device memory (GLOBAL
// true; any size, walk of step 1, every slot on it).  Per round, the
// survivors whose CAS inserted a key take the next ids (thread order).
// Writes the bin's distinct keys to ustage[start + id] and each survivor's
// id to tu_l[its tile slot].  Returns false (the LDS pass only) once the bin
// has more than `max_keys` distinct keys; the caller then redoes the bin.
// A key that finds the LDS set full can only do so past that limit.  Key -1,
// the empty marker, is carried in s_neg.
template <bool GLOBAL>
__device__ bool bin_pass(const u32x4* __restrict__ ent, int64_t start, int cnt, unsigned long long* skeys,
                         int32_t* sids, uint32_t size, int max_keys, int32_t* __restrict__ tu_l,
                         int64_t* __restrict__ ustage, int* s_wave, int* s_neg, int* nd_out) {
    const int tid = threadIdx.x;
    int nd = 0;
    if (tid == 0) {
        s_neg[0] = 0;    // key -1 claimed
        s_neg[1] = -1;   // its id
    }
    __syncthreads();
    for (int r0 = 0; r0 < cnt; r0 += kBinThreads * kBinVec) {
        uint64_t k[kBinVec];
        int32_t org[kBinVec];
        uint32_t q[kBinVec];
        uint32_t valid = 0, won = 0;
        // the round's entries are loaded without a branch each (past the
        // bin's end its last entry is loaded again and ignored), so the
        // loads are in flight together
        u32x4 v[kBinVec];
#pragma unroll
        for (int u = 0; u < kBinVec; ++u) {
            const int e = r0 + u * kBinThreads + tid;
            v[u] = ent[start + (e < cnt ? e : cnt - 1)];
        }
#pragma unroll
        for (int u = 0; u < kBinVec; ++u) {
            const int e = r0 + u * kBinThreads + tid;
            k[u] = 0;
            org[u] = 0;
            q[u] = 0;
            if (e < cnt) {
                k[u] = ((uint64_t)v[u].y << 32) | v[u].x;
                org[u] = (int32_t)v[u].z;
                valid |= 1u << u;
            }
        }
#pragma unroll
        for (int u = 0; u < kBinVec; ++u) {
            if (!(valid & (1u << u))) continue;
            if (k[u] == kFree) {
                if (atomicCAS(&s_neg[0], 0, 1) == 0) won |= 1u << u;
                continue;
            }
            const uint64_t h = mix64(k[u] ^ kSalt1);
            uint32_t p, stp;
            if (GLOBAL) {
                p = (uint32_t)(h % size);
                stp = 1;
            } else {
                p = (uint32_t)h & (size - 1);
                stp = ((uint32_t)(h >> 32) | 1u) & (size - 1);
            }
            for (uint32_t probe = 0; probe < size; ++probe) {
                const unsigned long long old = atomicCAS(&skeys[p], kFree, (unsigned long long)k[u]);
                if (old == kFree) {
                    won |= 1u << u;
                    break;
                }
                if (old == k[u]) break;
                p += stp;
                if (GLOBAL) p = p >= size ? p - size : p;
                else p &= size - 1;
            }
            q[u] = p;
        }
        int tot;
        int id = nd + bin_block_scan(__popc(won), s_wave, &tot);
        if (!GLOBAL && nd + tot > max_keys) return false;   // tot is the same in every thread
#pragma unroll
        for (int u = 0; u < kBinVec; ++u) {
            if (!(won & (1u << u))) continue;
            if (k[u] == kFree) s_neg[1] = id;
            else sids[q[u]] = id;
            ustage[start + id] = (int64_t)k[u];
            ++id;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kBinVec; ++u) {
            if (!(valid & (1u << u))) continue;
            int32_t v;
            if (k[u] == kFree) v = s_neg[1];
            else if (GLOBAL) v = __hip_atomic_load(&sids[q[u]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else v = sids[q[u]];
            tu_l[org[u]] = v;
        }
        nd += tot;
    }
    *nd_out = nd;
    return true;
}

// One workgroup per bin: the LDS set first; a bin that outgrows it is redone
// in its own region of fb_keys / fb_ids (2*cnt + 1 slots from 2*start + bin,
// so the regions of the bins do not overlap).
__global__ __launch_bounds__(kBinThreads) void k_part_dedup(const u32x4* __restrict__ ent,
                                                           const int32_t* __restrict__ total,
                                                           int32_t* __restrict__ base, int max_keys,
                                                           int32_t* __restrict__ tu_l,
                                                           int64_t* __restrict__ ustage,
                                                           int32_t* __restrict__ ucount,
                                                           unsigned long long* __restrict__ fb_keys,
                                                           int32_t* __restrict__ fb_ids) {
    __shared__ unsigned long long s_key[kBinSet];
    __shared__ int32_t s_id[kBinSet];
    __shared__ int s_wave[kBinThreads / 64];
    __shared__ int s_neg[2];
    const int b = blockIdx.x;
    // the bin's start: survivors of the bins before it
    constexpr int kPer = (1 << kPartMaxLog2) / kBinThreads;
    int part = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = threadIdx.x * kPer + u;
        part += i < b ? total[i] : 0;
    }
    for (int i = threadIdx.x; i < kBinSet; i += kBinThreads) s_key[i] = kFree;
    int start32;
    bin_block_scan(part, s_wave, &start32);   // its barriers also order the set clear
    const int64_t start = start32;
    const int cnt = total[b];
    if (threadIdx.x == 0) base[b] = start32;
    int nd = 0;
    if (!bin_pass<false>(ent, start, cnt, s_key, s_id, kBinSet, max_keys, tu_l, ustage, s_wave, s_neg, &nd)) {
        const int64_t fb0 = 2 * start + b;
        const uint32_t size = 2u * (uint32_t)cnt + 1u;
        for (uint32_t i = threadIdx.x; i < size; i += kBinThreads) fb_keys[fb0 + i] = kFree;
        __syncthreads();
        bin_pass<true>(ent, start, cnt, fb_keys + fb0, fb_ids + fb0, size, cnt, tu_l, ustage, s_wave, s_neg,
                       &nd);
    }
    if (threadIdx.x == 0) ucount[b] = nd;
}

// Blocks [0, pack_blocks) (pack_blocks is 0 or the number of bins): pack bin
// b's distinct keys at uoff[b]; the other blocks: compose the inverse tile
// by tile, id = uoff[bin] + id inside the bin.  With `slots` (the
// find-or-insert result of `unique`), each survivor also fetches its key's
// slot once into LDS and sid[i] = slots[inverse[i]] is written beside the
// inverse (one index per ID, in sequence, for a later gather).
__global__ __launch_bounds__(kTileThreads) void k_part_finish(
    const int64_t* __restrict__ ustage, const int32_t* __restrict__ base, int plog2,
    const int32_t* __restrict__ ucount, const int32_t* __restrict__ uoff, int64_t* __restrict__ unique,
    int64_t* __restrict__ n_unique, const int64_t* __restrict__ tu_keys, const int32_t* __restrict__ tu_count,
    const int32_t* __restrict__ tu_l, const uint16_t* __restrict__ local, int64_t n,
    int32_t* __restrict__ inverse, int pack_blocks, const int32_t* __restrict__ slots,
    int32_t* __restrict__ sid) {
    const int P = 1 << plog2;
    if ((int)blockIdx.x < pack_blocks) {
        const int b = blockIdx.x;
        const int64_t src = base[b];
        const int64_t dst = uoff[b];
        const int c = ucount[b];
        for (int l = threadIdx.x; l < c; l += kTileThreads) unique[dst + l] = ustage[src + l];
        if (b == 0 && threadIdx.x == 0) *n_unique = uoff[P];
        return;
    }
    __shared__ int32_t s_gid[kTile];
    __shared__ int32_t s_sl[kTile];
    __shared__ int32_t s_uoff[1 << kPartMaxLog2];
    for (int b = threadIdx.x; b < P; b += kTileThreads) s_uoff[b] = uoff[b];
    __syncthreads();
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int64_t tile = (int64_t)blockIdx.x - pack_blocks; tile < ntiles; tile += (int64_t)gridDim.x - pack_blocks) {
        // loads without a branch per element (past the end the last
        // element is loaded again and dropped), so each pass's loads are in
        // flight together
        constexpr int kV = 4;
        const int cnt = tu_count[tile];
        for (int j0 = threadIdx.x; j0 < cnt; j0 += kV * kTileThreads) {
            uint64_t k[kV];
            int32_t l[kV];
#pragma unroll
            for (int u = 0; u < kV; ++u) {
                const int j = j0 + u * kTileThreads;
                const int64_t at = tile * kTile + (j < cnt ? j : cnt - 1);
                k[u] = (uint64_t)tu_keys[at];
                l[u] = tu_l[at];
            }
            int32_t g[kV];
#pragma unroll
            for (int u = 0; u < kV; ++u) g[u] = s_uoff[part_bin(k[u], plog2)] + l[u];
            if (slots) {
                int32_t sl[kV];
#pragma unroll
                for (int u = 0; u < kV; ++u) sl[u] = slots[g[u]];
#pragma unroll
                for (int u = 0; u < kV; ++u) {
                    const int j = j0 + u * kTileThreads;
                    if (j < cnt) s_sl[j] = sl[u];
                }
            }
#pragma unroll
            for (int u = 0; u < kV; ++u) {
                const int j = j0 + u * kTileThreads;
                if (j < cnt) s_gid[j] = g[u];
            }
        }
        __syncthreads();
        const int64_t b0 = tile * kTile;
        constexpr int kPerT = kTile / kTileThreads;
        uint16_t lo[kPerT];
#pragma unroll
        for (int u = 0; u < kPerT; ++u) {
            const int64_t i = b0 + u * kTileThreads + threadIdx.x;
            const int64_t ic = i < n ? i : n - 1;
            lo[u] = local ? local[ic] : (uint16_t)(ic - b0);   // no stage 1: every ID is its own survivor
        }
#pragma unroll
        for (int u = 0; u < kPerT; ++u) {
            const int64_t i = b0 + u * kTileThreads + threadIdx.x;
            if (i < n) {
                inverse[i] = s_gid[lo[u]];
                if (slots) sid[i] = s_sl[lo[u]];
            }
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

size_t dedup_workspace_bytes(int64_t n) {
    if (n < 0) n = 0;
    size_t b = layout(n, nullptr).bytes;
    if (n > kTile && n <= kPartMaxN) {
        const size_t bp = part_layout(n, nullptr).bytes;
        if (bp > b) b = bp;
    }
    return b;
}

}  // extern "C"

// Stage-2 forms.  The default for a batch (N-based, and what the adaptive
// call starts from): one tile -> kOneTile; unordered 2^11 < n <= 2^23 ->
// kBins; the ordered mode and larger batches -> kSet.  HTL_DEDUP_PATH
// forces a form where it applies: "set" (any size), "bins" / "bins_only"
// (unordered 2^11 < n <= 2^23).  HTL_DEDUP_BIN_MAX lowers the distinct keys
// a bin may hold in LDS (to test the device-memory redo).
enum DedupPath { kOneTile = HTL_DEDUP_ONE_TILE, kBins = HTL_DEDUP_TWO_STAGE_BINS, kBinsOnly = HTL_DEDUP_BINS_ONLY,
                 kSet = HTL_DEDUP_DEVICE_SET };

static bool bins_allowed(bool ordered, int64_t n) { return !ordered && n > kTile && n <= kPartMaxN; }

static int default_path(bool ordered, int64_t n) {
    if (n <= kTile) return kOneTile;
    return bins_allowed(ordered, n) ? kBins : kSet;
}

static int forced_path(bool ordered, int64_t n, int chosen) {
    if (n <= kTile) return kOneTile;
    const char* e = getenv("HTL_DEDUP_PATH");
    if (!e) return chosen;
    const std::string v(e);
    if (v == "set") return kSet;
    if (bins_allowed(ordered, n) && v == "bins") return kBins;
    if (bins_allowed(ordered, n) && v == "bins_only") return kBinsOnly;
    return chosen;
}

static int bin_max_keys() {
    const char* e = getenv("HTL_DEDUP_BIN_MAX");
    if (!e) return kBinMax;
    const int v = atoi(e);
    return v < 0 ? 0 : (v > kBinMax ? kBinMax : v);
}

// Statistics of one call, for the adaptive choice of the next: written by
// one workgroup at the end of the call into pinned host memory (seqlock:
// seq odd while the fields are being written).
struct DedupStatsDev {
    volatile int64_t seq;
    volatile int64_t n;
    volatile int64_t survivors;
    volatile int64_t n_unique;
    volatile int64_t path;
};

// survivors: the sum of per-tile counts (stage 1), or n (no stage 1).
__global__ __launch_bounds__(1024) void k_dedup_stats(DedupStatsDev* st, int64_t call, int64_t n, int path,
                                                      const int32_t* __restrict__ tu_count, int64_t ntiles,
                                                      const int64_t* __restrict__ n_unique) {
    __shared__ int64_t s_part[1024 / 64];
    int64_t sum = 0;
    if (tu_count)
        for (int64_t t = threadIdx.x; t < ntiles; t += 1024) sum += tu_count[t];
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane_id() == 0) s_part[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t tot = 0;
        for (int w = 0; w < 1024 / 64; ++w) tot += s_part[w];
        const int64_t u = *n_unique;
        st->seq = 2 * call - 1;
        __threadfence_system();
        st->n = n;
        st->survivors = tu_count ? tot : (path == kOneTile ? u : n);
        st->n_unique = u;
        st->path = path;
        __threadfence_system();
        st->seq = 2 * call;
    }
}

struct StatsSink {
    DedupStatsDev* dev = nullptr;
    int64_t call = 0;
};

static htl_status run_part(const char* who, const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                           int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream, DedupRun* split,
                           bool raw, const StatsSink& sink) {
    PartWs w = part_layout(n, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, std::string(who) + ": workspace too small");
    const int64_t ntiles = ceil_div(n, kTile);
    const int P = 1 << w.plog2;
    const size_t bin_lds = (size_t)P * 4;
    const unsigned gt = grid_for(ntiles, 1, 1 << 16);
    static_assert((1 << kPartMaxLog2) <= 4 * kBaseThreads, "one-workgroup bin prefix");
    // raw: no stage 1 -- the tiles' survivors are their keys, in place
    const int64_t* tkeys = raw ? keys : w.tu_keys;
    const uint16_t* local = raw ? nullptr : w.local;
    if (raw)
        hipLaunchKernelGGL(k_tile_lengths, dim3(grid_for(ntiles, 256)), dim3(256), 0, stream, w.tu_count, n, ntiles);
    else
        hipLaunchKernelGGL(k_dedup_tile<false>, dim3(gt), dim3(kTileThreads), 0, stream, keys, n, w.tu_keys,
                           w.tu_count, w.local, (int32_t*)nullptr, (int64_t*)nullptr, SetClear{});
    hipLaunchKernelGGL(k_part_count, dim3(w.rows), dim3(kRowThreads), bin_lds, stream, tkeys, w.tu_count, ntiles,
                       w.tpr, w.plog2, w.cnt);
    hipLaunchKernelGGL(k_col_scan, dim3(P / kColBins), dim3(1024), 0, stream, w.cnt, w.rows, w.plog2, w.btotal);
    hipLaunchKernelGGL(k_part_scatter, dim3(w.rows), dim3(kRowThreads), bin_lds, stream, tkeys, w.tu_count,
                       ntiles, w.cnt, w.btotal, w.rows, w.tpr, w.plog2, w.ent);
    hipLaunchKernelGGL(k_part_dedup, dim3(P), dim3(kBinThreads), 0, stream, w.ent, w.btotal, w.base, bin_max_keys(),
                       w.tu_l, w.ustage, w.ucount, w.fb_keys, w.fb_ids);
    hipLaunchKernelGGL(k_prefix_bins, dim3(1), dim3(kBaseThreads), 0, stream, w.ucount, P, w.uoff);
    // packing the bins' keys and composing the inverse share one launch;
    // split: the packing only (the compose runs after find-or-insert)
    const unsigned grid = split ? P : P + gt;
    hipLaunchKernelGGL(k_part_finish, dim3(grid), dim3(kTileThreads), 0, stream, w.ustage, w.base, w.plog2,
                       w.ucount, w.uoff, unique, n_unique_dev, tkeys, w.tu_count, w.tu_l, local, n, inverse, P,
                       (const int32_t*)nullptr, (int32_t*)nullptr);
    if (sink.dev)
        hipLaunchKernelGGL(k_dedup_stats, dim3(1), dim3(1024), 0, stream, sink.dev, sink.call, n,
                           raw ? (int)kBinsOnly : (int)kBins, raw ? (const int32_t*)nullptr : w.tu_count, ntiles,
                           (const int64_t*)n_unique_dev);
    if (split) *split = DedupRun{kRunPart, n, ws, raw ? keys : nullptr};
    return check_launch(who);
}

static htl_status run_dedup(const char* who, bool ordered, const int64_t* keys, int64_t n, int64_t* unique,
                            int32_t* inverse, int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream,
                            DedupRun* split = nullptr, int path = -1, const StatsSink& sink = StatsSink{}) {
    clear_error();
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 30), std::string(who) + ": n must be in [0, 2^30)");
    HTL_REQUIRE(n_unique_dev && aligned(n_unique_dev, 8), std::string(who) + ": null or misaligned n_unique_dev");
    if (split) *split = DedupRun{kRunDone, n, ws, nullptr};
    if (n == 0) {
        hipLaunchKernelGGL(k_write_zero, dim3(1), dim3(1), 0, stream, n_unique_dev);
        return check_launch(who);
    }
    HTL_REQUIRE(keys && unique && inverse && ws, std::string(who) + ": null pointer");
    HTL_REQUIRE(aligned(keys, 8) && aligned(unique, 8) && aligned(inverse, 4) && aligned(ws, 256),
                std::string(who) + ": misaligned pointer");
    if (path < 0) path = default_path(ordered, n);
    path = forced_path(ordered, n, path);
    if (path == kBins || path == kBinsOnly)
        return run_part(who, keys, n, unique, inverse, n_unique_dev, ws, ws_bytes, stream, split, path == kBinsOnly,
                        sink);
    DedupWs w = layout(n, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, std::string(who) + ": workspace too small");
    if (path == kOneTile) {
        // A batch of one tile: the LDS stage alone is the answer (one
        // launch, no device set to clear), in first-occurrence order, which
        // both modes accept.  Nothing is left for a split's second half.
        hipLaunchKernelGGL(k_dedup_tile<true>, dim3(1), dim3(kTileThreads), 0, stream, keys, n, unique,
                           (int32_t*)nullptr, (uint16_t*)nullptr, inverse, n_unique_dev, SetClear{});
        if (sink.dev)
            hipLaunchKernelGGL(k_dedup_stats, dim3(1), dim3(1024), 0, stream, sink.dev, sink.call, n, (int)kOneTile,
                               (const int32_t*)nullptr, (int64_t)1, (const int64_t*)n_unique_dev);
        return check_launch(who);
    }
    const int64_t ntiles = ceil_div(n, kTile);
    const unsigned gt = grid_for(ntiles, 1, 1 << 16);
    // the stage-1 grid also clears the device set (owners only in ordered mode)
    const SetClear clr{w.set_keys, ordered ? w.set_owner : nullptr, w.cap, w.misc};
    hipLaunchKernelGGL(k_dedup_tile<false>, dim3(gt), dim3(kTileThreads), 0, stream, keys, n, w.tu_keys, w.tu_count,
                       w.local, (int32_t*)nullptr, (int64_t*)nullptr, clr);
    if (ordered) {
        hipLaunchKernelGGL(k_dedup_claim<true>, dim3(gt), dim3(kGlobalThreads), 0, stream, w.tu_keys, w.tu_count,
                           ntiles, w.set_keys, w.set_owner, (uint64_t)(w.cap - 1), w.tu_slot, w.tu_own, w.tile_win,
                           w.misc);
        hipLaunchKernelGGL(k_dedup_count, dim3(gt), dim3(kGlobalThreads), 0, stream, w.tu_count, w.tu_slot, ntiles,
                           w.set_owner, w.tile_win);
    } else {
        hipLaunchKernelGGL(k_dedup_claim<false>, dim3(gt), dim3(kGlobalThreads), 0, stream, w.tu_keys, w.tu_count,
                           ntiles, w.set_keys, w.set_owner, (uint64_t)(w.cap - 1), w.tu_slot, w.tu_own, w.tile_win,
                           w.misc);
    }
    htl_status st = scan_exclusive_i32(w.tile_win, w.tile_off, ntiles, nullptr, kScanIdentity, 1, w.scan_tmp, stream);
    if (st != HTL_OK) return st;
    if (ordered)
        hipLaunchKernelGGL(k_dedup_assign<true>, dim3(gt), dim3(kGlobalThreads), 0, stream, w.tu_keys, w.tu_count,
                           w.tu_slot, w.tu_own, ntiles, w.set_owner, w.tile_off, w.set_ids, unique, n_unique_dev);
    else
        hipLaunchKernelGGL(k_dedup_assign<false>, dim3(gt), dim3(kGlobalThreads), 0, stream, w.tu_keys, w.tu_count,
                           w.tu_slot, w.tu_own, ntiles, w.set_owner, w.tile_off, w.set_ids, unique, n_unique_dev);
    if (sink.dev)
        hipLaunchKernelGGL(k_dedup_stats, dim3(1), dim3(1024), 0, stream, sink.dev, sink.call, n, (int)kSet,
                           (const int32_t*)w.tu_count, ntiles, (const int64_t*)n_unique_dev);
    if (split) {
        *split = DedupRun{kRunSet, n, ws, nullptr};
        return check_launch(who);
    }
    hipLaunchKernelGGL(k_dedup_compose, dim3(gt), dim3(kTileThreads), 0, stream, w.local, n, w.tu_count, w.tu_slot,
                       w.set_ids, inverse, (const int32_t*)nullptr, (int32_t*)nullptr);
    return check_launch(who);
}

namespace htl {

htl_status dedup_until_unique(const char* who, const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                              int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream, DedupRun* run) {
    return run_dedup(who, false, keys, n, unique, inverse, n_unique_dev, ws, ws_bytes, stream, run);
}

htl_status dedup_compose(const char* who, const DedupRun& run, const int32_t* slots, int32_t* inverse, int32_t* sid,
                         hipStream_t stream) {
    if (run.path == kRunDone) return HTL_OK;
    const int64_t n = run.n;
    const int64_t ntiles = ceil_div(n, kTile);
    const unsigned gt = grid_for(ntiles, 1, 1 << 16);
    if (run.path == kRunPart) {
        PartWs w = part_layout(n, (char*)run.ws);
        // raw_keys: no stage 1 ran; the survivors are the keys themselves
        const int64_t* tkeys = run.raw_keys ? run.raw_keys : w.tu_keys;
        const uint16_t* local = run.raw_keys ? nullptr : w.local;
        hipLaunchKernelGGL(k_part_finish, dim3(gt), dim3(kTileThreads), 0, stream, w.ustage, w.base, w.plog2,
                           w.ucount, w.uoff, (int64_t*)nullptr, (int64_t*)nullptr, tkeys, w.tu_count, w.tu_l, local,
                           n, inverse, 0, slots, sid);
    } else {
        DedupWs w = layout(n, (char*)run.ws);
        hipLaunchKernelGGL(k_dedup_compose, dim3(gt), dim3(kTileThreads), 0, stream, w.local, n, w.tu_count,
                           w.tu_slot, w.set_ids, inverse, slots, sid);
    }
    return check_launch(who);
}

}  // namespace htl

// ------------------------------------------------------- adaptive unique --
// The TensorFlow article's section 3.6: a heuristic picks the Unique
// implementation.  Here the plan remembers the statistics of its previous
// calls (written by the device into pinned host memory at the end of each
// call, read by the host at the next call without waiting for the device),
// and picks the stage-2 form from the batch size and the duplicates that
// stage 1 found in the last measured batch:
//   n <= 2^11                 one tile (one launch);
//   2^11 < n <= 2^23          hash bins, without stage 1 when too few
//                             duplicates were found for any key to overfill
//                             a bin, else with it;
//   n > 2^23                  the device-wide set.
// Why that bound: stage 1 keeps one copy of a key per tile, so it removes at
// least c - ntiles copies of a key that occurs c times; a measured duplicate
// share d = (n - survivors) / n therefore bounds the hottest key by
// d n + ntiles.  Without stage 1 every copy of a key lands in its one bin,
// whose workgroup dedups them in turn; stage 1 is skipped only while
// d n + ntiles <= 3 n / P (P bins), so no key can bring a bin past about
// four times the mean load.  (On the sweep of hash_table_lookup_amd.tune:
// skipping saves up to 15% at 2^20..2^23 keys when the tiles hold almost no
// duplicates, and costs 3-14x under Zipf skew, where a hot key fills one bin.)
// A batch run without stage 1 cannot measure d, so while the plan skips it,
// every kRemeasure-th call runs both stages again to renew the measurement.
struct htl_dedup_plan {
    DedupStatsDev* host = nullptr;   // pinned, mapped
    DedupStatsDev* dev = nullptr;    // its device address
    int64_t calls = 0;               // calls enqueued with statistics
    mutable double dup = -1.0;       // last measured (n - survivors) / n (-1: none yet)
    mutable int64_t kept_call = 0;   // the call that measured it
    int device = -1;
};

namespace {
constexpr int64_t kRemeasure = 8;
}

extern "C" {

htl_status dedup_unique_inverse(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    const htl_status st =
        run_dedup("dedup_unique_inverse", false, keys, n, unique, inverse, n_unique_dev, ws, ws_bytes, stream);
    if (st == HTL_OK) debug_check_dedup(keys, n, unique, inverse, n_unique_dev, stream);
    return st;
}

htl_status dedup_unique_inverse_ordered(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                        int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    const htl_status st = run_dedup("dedup_unique_inverse_ordered", true, keys, n, unique, inverse, n_unique_dev, ws,
                                    ws_bytes, stream);
    if (st == HTL_OK) debug_check_dedup(keys, n, unique, inverse, n_unique_dev, stream);
    return st;
}

htl_status dedup_plan_create(htl_dedup_plan** plan) {
    clear_error();
    HTL_REQUIRE(plan != nullptr, "dedup_plan_create: null plan");
    *plan = nullptr;
    htl_dedup_plan* p = new (std::nothrow) htl_dedup_plan();
    if (!p) return fail(HTL_ERR_NOMEM, "dedup_plan_create: out of host memory");
    void* h = nullptr;
    if (hipHostMalloc(&h, sizeof(DedupStatsDev), hipHostMallocMapped) != hipSuccess || !h) {
        delete p;
        return fail(HTL_ERR_NOMEM, "dedup_plan_create: hipHostMalloc of the statistics failed");
    }
    std::memset(h, 0, sizeof(DedupStatsDev));
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || !d) {
        (void)hipHostFree(h);
        delete p;
        return fail(HTL_ERR_DEVICE, "dedup_plan_create: no device address for the pinned statistics");
    }
    p->host = (DedupStatsDev*)h;
    p->dev = (DedupStatsDev*)d;
    (void)hipGetDevice(&p->device);
    *plan = p;
    return HTL_OK;
}

htl_status dedup_plan_destroy(htl_dedup_plan* plan) {
    clear_error();
    if (!plan) return HTL_OK;
    // the device may still write the statistics of an enqueued call
    HTL_HIP(hipDeviceSynchronize());
    (void)hipHostFree(plan->host);
    delete plan;
    return HTL_OK;
}

htl_status dedup_plan_stats(const htl_dedup_plan* plan, htl_dedup_stats* out) {
    clear_error();
    HTL_REQUIRE(plan && out, "dedup_plan_stats: null argument");
    // seqlock read of what the device last wrote (no wait for the device)
    for (int attempt = 0; attempt < 64; ++attempt) {
        const int64_t s1 = plan->host->seq;
        if (s1 & 1) continue;
        std::atomic_thread_fence(std::memory_order_acquire);
        htl_dedup_stats v;
        v.calls = s1 / 2;
        v.n = plan->host->n;
        v.survivors = plan->host->survivors;
        v.n_unique = plan->host->n_unique;
        v.path = (int32_t)plan->host->path;
        std::atomic_thread_fence(std::memory_order_acquire);
        if (plan->host->seq == s1) {
            *out = v;
            return HTL_OK;
        }
    }
    *out = htl_dedup_stats{};   // being written: report nothing seen yet
    return HTL_OK;
}

int32_t dedup_plan_choose(const htl_dedup_plan* plan, int64_t n) {
    if (n <= kTile) return kOneTile;
    if (n > kPartMaxN) return kSet;
    if (!plan) return kBins;
    htl_dedup_stats v{};
    if (dedup_plan_stats(plan, &v) == HTL_OK && v.calls > plan->kept_call && v.n > 0 && v.path != kBinsOnly) {
        plan->dup = (double)(v.n - v.survivors) / (double)v.n;    // a fresh measurement of stage 1
        plan->kept_call = v.calls;
    }
    if (plan->dup < 0) return kBins;
    const double P = (double)((int64_t)1 << part_layout(n, nullptr).plog2);
    const double ntiles = (double)ceil_div(n, kTile);
    if (plan->dup * (double)n + ntiles > 3.0 * (double)n / P) return kBins;
    // skipping stage 1: every kRemeasure-th call measures it again
    return ((plan->calls + 1) % kRemeasure == 0) ? kBins : kBinsOnly;
}

htl_status dedup_unique_inverse_adaptive(htl_dedup_plan* plan, const int64_t* keys, int64_t n, int64_t* unique,
                                         int32_t* inverse, int64_t* n_unique_dev, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(plan != nullptr, "dedup_unique_inverse_adaptive: null plan");
    const int path = dedup_plan_choose(plan, n);
    StatsSink sink{plan->dev, plan->calls + 1};
    const htl_status st = run_dedup("dedup_unique_inverse_adaptive", false, keys, n, unique, inverse, n_unique_dev,
                                    ws, ws_bytes, stream, nullptr, path, n > 0 ? sink : StatsSink{});
    if (st == HTL_OK && n > 0) ++plan->calls;
    if (st == HTL_OK) debug_check_dedup(keys, n, unique, inverse, n_unique_dev, stream);
    return st;
}

}  // extern "C"
