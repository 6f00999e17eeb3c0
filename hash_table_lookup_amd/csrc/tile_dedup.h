// Stage 1 of the feature-ID dedup: one workgroup dedups one tile of keys in
// LDS (internal header of the dedup).
//
// MTGenRec (arXiv 2505.12663) TL;DR: two-stage ID deduplication; MTGR (arXiv
// 2505.18654) section 5, "Embedding Lookup": IDs are unique before the
// exchange.  One copy of each key leaves the tile.
#pragma once

#include "htl_common.h"

namespace htl {
namespace {

constexpr int kTile = 2048;            // keys per stage-1 tile
constexpr int kTileLog2 = 11;
// Threads per tile (and per block of the tile-wise stage-2 kernels).  The
// tile's LDS (48 KB) allows three blocks per CU: 512 threads keep 24 waves
// per CU in flight.  Large-table step 0.608 / 0.597 / 0.602 ms and
// merged-tables step 2.771 / 2.759 / 2.814 ms with 256 / 512 / 1024.
constexpr int kTileThreads = 512;
constexpr int kKeysPerThread = kTile / kTileThreads;
constexpr int kLdsCap = 2 * kTile;     // LDS set slots (load <= 1/2); slot kLdsCap holds key -1
constexpr int kLdsCapLog2 = kTileLog2 + 1;
constexpr uint64_t kFree = ~0ull;      // empty marker of both sets (key -1 is out of band)
constexpr uint64_t kSalt1 = 0x6A09E667F3BCC909ull;
constexpr uint64_t kSalt2 = 0xBB67AE8584CAA73Bull;
constexpr int kNoOwner = 0x7FFFFFFF;

// Block-wide exclusive prefix count of `flag` over the block's threads in
// thread order; returns this thread's prefix and leaves the block total in
// *total.  Uses s_wave[kTileThreads / 64].
__device__ __forceinline__ int block_rank(bool flag, int* s_wave, int* total) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    const uint64_t m = __ballot(flag);
    if (lane == 0) s_wave[wid] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTileThreads / 64; ++w) {
        const int c = s_wave[w];
        before += (w < wid) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return before + __popcll(m & lanemask_lt());
}

// The device set of stage 2, cleared by the stage-1 grid before its tiles
// (the stores stream out while the tiles work in LDS; stage 2 starts after
// the whole grid).  keys == nullptr: nothing to clear.
struct SetClear {
    unsigned long long* keys;   // [cap] -> kFree
    int32_t* owner;             // [cap + 1] -> kNoOwner, or nullptr
    uint64_t cap;               // a power of two >= 256
    int32_t* misc;              // misc[0] -> 0
};

__device__ __forceinline__ void clear_set(const SetClear& c) {
    typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    u64x2 f;
    f.x = f.y = kFree;
    u64x2* k2 = reinterpret_cast<u64x2*>(c.keys);
    for (int64_t i = t0; i < (int64_t)(c.cap / 2); i += stride) k2[i] = f;
    if (c.owner)
        for (int64_t i = t0; i <= (int64_t)c.cap; i += stride) c.owner[i] = kNoOwner;
    if (t0 == 0) c.misc[0] = 0;
}

// Hash bin of a key in the partitioned stage 2: the top plog2 bits of a
// salted mix (the LDS sets inside a bin hash with the other salt).
__device__ __forceinline__ uint32_t part_bin(uint64_t k, int plog2) {
    return (uint32_t)(mix64(k ^ kSalt2) >> (64 - plog2));
}

// Stage 1: dedup one tile in LDS.  Tile-local ids follow the order of first
// occurrence inside the tile (LDS atomicMin of the position, then a block
// scan over positions), so the result does not depend on scheduling.
// FINAL (a batch of at most one tile, one workgroup): the tile's result is
// the whole answer, written straight to unique / inverse / the unique count
// (tu_keys, local, tu_count stand for them), in first-occurrence order.
template <bool FINAL>
__global__ __launch_bounds__(kTileThreads) void k_dedup_tile(const int64_t* __restrict__ keys, int64_t n,
                                                            int64_t* __restrict__ tu_keys,
                                                            int32_t* __restrict__ tu_count,
                                                            uint16_t* __restrict__ local,
                                                            int32_t* __restrict__ inverse,
                                                            int64_t* __restrict__ n_unique, SetClear clr) {
    __shared__ unsigned long long s_key[kLdsCap];
    __shared__ int32_t s_tag[kLdsCap + 1];   // first position of the key, then its tile-local id
    __shared__ int s_jcnt[kKeysPerThread][kTileThreads / 64];
    const int tid = threadIdx.x;
    if (!FINAL && clr.keys) clear_set(clr);

    for (int64_t tile = blockIdx.x; tile * kTile < n; tile += gridDim.x) {
        const int64_t base = tile * kTile;
        // the tile's keys are requested first, so that they arrive while the
        // LDS set is being cleared
        uint64_t k[kKeysPerThread];
        int pos[kKeysPerThread];
        uint32_t valid = 0;
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            const int64_t idx = base + j * kTileThreads + tid;
            k[j] = 0;
            pos[j] = 0;
            if (idx < n) {
                valid |= 1u << j;
                k[j] = (uint64_t)keys[idx];
            }
        }
        for (int i = tid; i < kLdsCap; i += kTileThreads) s_key[i] = kFree;
        for (int i = tid; i <= kLdsCap; i += kTileThreads) s_tag[i] = kTile;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            if (!(valid & (1u << j))) continue;
            int p = kLdsCap;                         // key -1: out of band
            if (k[j] != kFree) {
                const uint64_t h = mix64(k[j] ^ kSalt1);
                uint32_t q = (uint32_t)(h >> (64 - kLdsCapLog2));
                const uint32_t stp = ((uint32_t)h | 1u) & (kLdsCap - 1);
                for (int probe = 0; probe < kLdsCap; ++probe) {
                    const unsigned long long old = atomicCAS(&s_key[q], kFree, (unsigned long long)k[j]);
                    if (old == kFree || old == k[j]) break;
                    q = (q + stp) & (kLdsCap - 1);
                }
                p = (int)q;
            }
            pos[j] = p;
            atomicMin(&s_tag[p], j * kTileThreads + tid);
        }
        __syncthreads();
        uint32_t first = 0;
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j)
            if ((valid & (1u << j)) && s_tag[pos[j]] == j * kTileThreads + tid) first |= 1u << j;
        __syncthreads();
        // ids in position order: positions j*kTileThreads + tid run j-major.  One
        // ballot per j; the per-wave counts of every j go through LDS at once.
        uint64_t bal[kKeysPerThread];
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            bal[j] = __ballot((first >> j) & 1u);
            if (lane_id() == 0) s_jcnt[j][tid >> 6] = __popcll(bal[j]);
        }
        __syncthreads();
        int run = 0;
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            int before = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < kTileThreads / 64; ++w) {
                const int c = s_jcnt[j][w];
                before += (w < (tid >> 6)) ? c : 0;
                tot += c;
            }
            if ((first >> j) & 1u) {
                const int id = run + before + __popcll(bal[j] & lanemask_lt());
                s_tag[pos[j]] = id;
                tu_keys[base + id] = (int64_t)k[j];
            }
            run += tot;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            if (!(valid & (1u << j))) continue;
            if (FINAL) inverse[base + j * kTileThreads + tid] = s_tag[pos[j]];
            else local[base + j * kTileThreads + tid] = (uint16_t)s_tag[pos[j]];
        }
        if (tid == 0) {
            if (FINAL) *n_unique = run;
            else tu_count[tile] = run;
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace htl
