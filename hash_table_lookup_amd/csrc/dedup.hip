// Two-stage feature-ID deduplication: unique keys plus inverse index.
//
// MTGenRec (arXiv 2505.12663), TL;DR and section 6 of its contents ("Embedding
// Table Lookup Acceleration"): two-stage ID deduplication for faster
// embedding lookups.  MTGR (arXiv 2505.18654) section 5, "Embedding Lookup":
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
// Adaptive choice (the TensorFlow article, section 3.6: a heuristic picks the
// Unique implementation): a batch of at most one tile (2048 keys, e.g. a
// serving request) is deduplicated by the LDS stage alone in one launch; the
// device set and its clear, the claim, the scan and the compose are skipped.
//
// Both sets probe with an odd step over a power-of-two capacity, so by
// MTGenRec's Theorem 1 a probe walk reaches every slot; with at most n keys in
// more than 3n/2 slots it always ends at a free slot (load at most 2/3: the
// set is cleared on every call, so its size is traded against that clear).
// The set is capped at 2^30 slots (its slot numbers, and the extra entry of
// key -1 at index 2^30, stay int32); with n < 2^30 a slot is always free.
// Every int64 is a valid key: the value -1, which both sets use as their
// empty marker, is carried out of band.
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
// own entry, the others' from the set), then maps its IDs.
__global__ __launch_bounds__(kTileThreads) void k_dedup_compose(const uint16_t* __restrict__ local, int64_t n,
                                                               const int32_t* __restrict__ tu_count,
                                                               const int32_t* __restrict__ tu_slot,
                                                               const int32_t* __restrict__ set_ids,
                                                               int32_t* __restrict__ inverse) {
    __shared__ int32_t s_gid[kTile];
    for (int64_t tile = blockIdx.x; tile * kTile < n; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        for (int j = threadIdx.x; j < cnt; j += kTileThreads) {
            const int32_t v = tu_slot[tile * kTile + j];
            s_gid[j] = v < 0 ? -(v + 1) : set_ids[v];
        }
        __syncthreads();
        const int64_t base = tile * kTile;
        for (int q = threadIdx.x; q < kTile; q += kTileThreads) {
            const int64_t i = base + q;
            if (i < n) inverse[i] = s_gid[local[i]];
        }
        __syncthreads();
    }
}

__global__ void k_write_zero(int64_t* p) { *p = 0; }

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

size_t dedup_workspace_bytes(int64_t n) {
    if (n < 0) n = 0;
    return layout(n, nullptr).bytes;
}

static htl_status run_dedup(const char* who, bool ordered, const int64_t* keys, int64_t n, int64_t* unique,
                            int32_t* inverse, int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 30), std::string(who) + ": n must be in [0, 2^30)");
    HTL_REQUIRE(n_unique_dev && aligned(n_unique_dev, 8), std::string(who) + ": null or misaligned n_unique_dev");
    if (n == 0) {
        hipLaunchKernelGGL(k_write_zero, dim3(1), dim3(1), 0, stream, n_unique_dev);
        return check_launch(who);
    }
    HTL_REQUIRE(keys && unique && inverse && ws, std::string(who) + ": null pointer");
    HTL_REQUIRE(aligned(keys, 8) && aligned(unique, 8) && aligned(inverse, 4) && aligned(ws, 256),
                std::string(who) + ": misaligned pointer");
    DedupWs w = layout(n, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, std::string(who) + ": workspace too small");
    if (n <= kTile) {
        // A batch of one tile: the LDS stage alone is the answer (one
        // launch, no device set to clear), in first-occurrence order, which
        // both modes accept.
        hipLaunchKernelGGL(k_dedup_tile<true>, dim3(1), dim3(kTileThreads), 0, stream, keys, n, unique,
                           (int32_t*)nullptr, (uint16_t*)nullptr, inverse, n_unique_dev, SetClear{});
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
    hipLaunchKernelGGL(k_dedup_compose, dim3(gt), dim3(kTileThreads), 0, stream, w.local, n, w.tu_count, w.tu_slot,
                       w.set_ids, inverse);
    return check_launch(who);
}

htl_status dedup_unique_inverse(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    return run_dedup("dedup_unique_inverse", false, keys, n, unique, inverse, n_unique_dev, ws, ws_bytes, stream);
}

htl_status dedup_unique_inverse_ordered(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                        int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    return run_dedup("dedup_unique_inverse_ordered", true, keys, n, unique, inverse, n_unique_dev, ws, ws_bytes,
                     stream);
}

}  // extern "C"
