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
//     distinct keys compactly to its own region, and a 16-bit local index per
//     key.  One copy of each key leaves the tile, as one copy per sender would
//     leave a device before the exchange; under Zipf traffic this also turns
//     the hottest key's thousands of global CASes into one per tile.
//   stage 2 (k_dedup_global): every tile survivor is inserted into a
//     device-wide open-addressing set (next_pow2(2n) slots, 64-bit CAS); the
//     winner of each key takes the next dense id.
//   compose (k_dedup_compose): inverse[i] = id(set slot of tile survivor
//     local[i]).
//
// Both sets probe with an odd step over a power-of-two capacity, so by
// MTGenRec's Theorem 1 a probe walk reaches every slot; with at most n keys in
// 2n slots it always ends at a free slot.  Every int64 is a valid key: the
// value -1, which both sets use as their empty marker, is carried out of band.
#include "htl_common.h"

namespace htl {
namespace {

constexpr int kTile = 2048;            // keys per stage-1 tile
constexpr int kTileLog2 = 11;
constexpr int kTileThreads = 256;
constexpr int kKeysPerThread = kTile / kTileThreads;
constexpr int kLdsCap = 2 * kTile;     // LDS set slots (load <= 1/2)
constexpr int kLdsCapLog2 = kTileLog2 + 1;
constexpr uint64_t kFree = ~0ull;      // empty marker of both sets (key -1 is out of band)
constexpr uint64_t kSalt1 = 0x6A09E667F3BCC909ull;
constexpr uint64_t kSalt2 = 0xBB67AE8584CAA73Bull;

struct DedupWs {
    unsigned long long* set_keys;   // [cap]
    int32_t* set_ids;               // [cap]
    int64_t* tu_keys;               // [ntiles * kTile]: per-tile distinct keys
    int32_t* tu_slot;               // [ntiles * kTile]: their set slot (-1: key -1)
    int32_t* tu_count;              // [ntiles]
    uint16_t* local;                // [n]
    int32_t* misc;                  // [0]: key -1 claimed, [1]: its dense id
    uint64_t cap;
    size_t bytes;
};

DedupWs layout(int64_t n, char* base) {
    DedupWs w{};
    const int64_t ntiles = ceil_div(n, kTile);
    uint64_t cap = 256;
    while (cap < (uint64_t)(2 * n)) cap <<= 1;
    w.cap = cap;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.set_keys = (unsigned long long*)take(cap * 8);
    w.set_ids = (int32_t*)take(cap * 4);
    w.tu_keys = (int64_t*)take((size_t)ntiles * kTile * 8);
    w.tu_slot = (int32_t*)take((size_t)ntiles * kTile * 4);
    w.tu_count = (int32_t*)take((size_t)ntiles * 4);
    w.local = (uint16_t*)take((size_t)n * 2);
    w.misc = (int32_t*)take(256);
    w.bytes = off;
    return w;
}

__global__ void k_dedup_clear(unsigned long long* __restrict__ set_keys, uint64_t cap,
                              unsigned long long* __restrict__ counter, int32_t* __restrict__ misc) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < (int64_t)cap; i += stride)
        set_keys[i] = kFree;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *counter = 0ull;
        misc[0] = 0;
        misc[1] = -1;
    }
}

__global__ __launch_bounds__(kTileThreads) void k_dedup_tile(const int64_t* __restrict__ keys, int64_t n,
                                                            int64_t* __restrict__ tu_keys,
                                                            int32_t* __restrict__ tu_count,
                                                            uint16_t* __restrict__ local) {
    __shared__ unsigned long long s_key[kLdsCap];
    __shared__ uint16_t s_id[kLdsCap];
    __shared__ int s_count, s_has_free_key, s_free_key_id;
    const int tid = threadIdx.x;
    const int lane = lane_id();

    for (int64_t tile = blockIdx.x; tile * kTile < n; tile += gridDim.x) {
        const int64_t base = tile * kTile;
        for (int i = tid; i < kLdsCap; i += kTileThreads) s_key[i] = kFree;
        if (tid == 0) {
            s_count = 0;
            s_has_free_key = 0;
        }
        __syncthreads();

        uint64_t k[kKeysPerThread];
        int pos[kKeysPerThread];
        uint32_t valid = 0, win = 0;
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
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            if (!(valid & (1u << j))) continue;
            if (k[j] == kFree) {                 // key -1: out of band
                pos[j] = kLdsCap;
                s_has_free_key = 1;
                continue;
            }
            const uint64_t h = mix64(k[j] ^ kSalt1);
            uint32_t p = (uint32_t)(h >> (64 - kLdsCapLog2));
            const uint32_t stp = ((uint32_t)h | 1u) & (kLdsCap - 1);
            for (int probe = 0; probe < kLdsCap; ++probe) {
                const unsigned long long old = atomicCAS(&s_key[p], kFree, (unsigned long long)k[j]);
                if (old == kFree) {
                    win |= 1u << j;
                    break;
                }
                if (old == k[j]) break;
                p = (p + stp) & (kLdsCap - 1);
            }
            pos[j] = (int)p;
        }
        __syncthreads();

        // Dense tile-local ids for the CAS winners: one LDS atomic per wavefront.
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            const bool w = (win >> j) & 1u;
            const uint64_t wm = __ballot(w);
            if (wm) {
                const int leader = __ffsll((unsigned long long)wm) - 1;
                int b = 0;
                if (lane == leader) b = atomicAdd(&s_count, __popcll(wm));
                b = __shfl(b, leader);
                if (w) {
                    const int id = b + __popcll(wm & lanemask_lt());
                    s_id[pos[j]] = (uint16_t)id;
                    tu_keys[base + id] = (int64_t)k[j];
                }
            }
        }
        __syncthreads();
        if (tid == 0 && s_has_free_key) {
            const int id = s_count++;
            s_free_key_id = id;
            tu_keys[base + id] = (int64_t)kFree;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kKeysPerThread; ++j) {
            if (!(valid & (1u << j))) continue;
            const int id = pos[j] == kLdsCap ? s_free_key_id : (int)s_id[pos[j]];
            local[base + j * kTileThreads + tid] = (uint16_t)id;
        }
        if (tid == 0) tu_count[tile] = s_count;
        __syncthreads();
    }
}

constexpr int kGlobalThreads = 256;

// Stage 2.  A slot is read before it is CASed: a key that is already in the
// set (the usual case for Zipf-hot keys, which every tile carries) costs a
// cacheable load instead of an atomic that would serialise with the same
// key's CAS from every other tile.  A CAS is attempted only on a slot seen
// EMPTY; if it loses, the value it returns decides (same key: found; other
// key: walk on).  Dense ids for the winners come from one atomicAdd per block
// iteration.
__global__ __launch_bounds__(kGlobalThreads) void k_dedup_global(
    const int64_t* __restrict__ tu_keys, const int32_t* __restrict__ tu_count, int64_t ntiles,
    unsigned long long* __restrict__ set_keys, int32_t* __restrict__ set_ids, uint64_t set_mask,
    int32_t* __restrict__ tu_slot, int64_t* __restrict__ unique, unsigned long long* __restrict__ counter,
    int32_t* __restrict__ misc) {
    __shared__ int s_wcnt[kGlobalThreads / 64];
    __shared__ unsigned long long s_base;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wid = tid >> 6;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        for (int jb = 0; jb < cnt; jb += kGlobalThreads) {
            const int j = jb + tid;
            const bool valid = j < cnt;
            uint64_t k = 0;
            bool win = false;
            int64_t slot = -1;
            if (valid) {
                k = (uint64_t)tu_keys[tile * kTile + j];
                if (k == kFree) {
                    if (__hip_atomic_load(&misc[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
                        win = atomicCAS(&misc[0], 0, 1) == 0;
                } else {
                    const uint64_t h = mix64(k ^ kSalt2);
                    uint64_t p = h & set_mask;
                    const uint64_t stp = ((h >> 32) | 1ull) & set_mask;
                    for (uint64_t probe = 0; probe <= set_mask; ++probe) {
                        const uint64_t cur = peek_u64(&set_keys[p]);
                        if (cur == k) break;
                        if (cur == kFree) {
                            const unsigned long long old = atomicCAS(&set_keys[p], kFree, (unsigned long long)k);
                            if (old == kFree) {
                                win = true;
                                break;
                            }
                            if (old == k) break;
                        }
                        p = (p + stp) & set_mask;
                    }
                    slot = (int64_t)p;
                }
            }
            const uint64_t wm = __ballot(win);
            if (lane == 0) s_wcnt[wid] = __popcll(wm);
            __syncthreads();
            if (tid == 0) {
                int run = 0;
                for (int w = 0; w < kGlobalThreads / 64; ++w) {
                    const int c = s_wcnt[w];
                    s_wcnt[w] = run;
                    run += c;
                }
                s_base = run ? atomicAdd(counter, (unsigned long long)run) : 0ull;
            }
            __syncthreads();
            if (win) {
                const int64_t gid = (int64_t)s_base + s_wcnt[wid] + __popcll(wm & lanemask_lt());
                unique[gid] = (int64_t)k;
                if (slot >= 0) set_ids[slot] = (int32_t)gid;
                else misc[1] = (int32_t)gid;
            }
            if (valid) tu_slot[tile * kTile + j] = (int32_t)slot;
            __syncthreads();
        }
    }
}

__global__ void k_dedup_compose(const uint16_t* __restrict__ local, int64_t n,
                                const int32_t* __restrict__ tu_slot, const int32_t* __restrict__ set_ids,
                                const int32_t* __restrict__ misc, int32_t* __restrict__ inverse) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t tile = i >> kTileLog2;
        const int32_t s = tu_slot[(tile << kTileLog2) + local[i]];
        inverse[i] = s >= 0 ? set_ids[s] : misc[1];
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

htl_status dedup_unique_inverse(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "dedup_unique_inverse: n must be in [0, 2^31)");
    HTL_REQUIRE(n_unique_dev && aligned(n_unique_dev, 8), "dedup_unique_inverse: null or misaligned n_unique_dev");
    if (n == 0) {
        hipLaunchKernelGGL(k_write_zero, dim3(1), dim3(1), 0, stream, n_unique_dev);
        return check_launch("dedup_unique_inverse");
    }
    HTL_REQUIRE(keys && unique && inverse && ws, "dedup_unique_inverse: null pointer");
    HTL_REQUIRE(aligned(keys, 8) && aligned(unique, 8) && aligned(inverse, 4) && aligned(ws, 256),
                "dedup_unique_inverse: misaligned pointer");
    DedupWs w = layout(n, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "dedup_unique_inverse: workspace too small");
    const int64_t ntiles = ceil_div(n, kTile);

    hipLaunchKernelGGL(k_dedup_clear, dim3(grid_for((int64_t)w.cap, 256 * 8, 1 << 14)), dim3(256), 0, stream,
                       w.set_keys, w.cap, (unsigned long long*)n_unique_dev, w.misc);
    hipLaunchKernelGGL(k_dedup_tile, dim3(grid_for(ntiles, 1, 1 << 16)), dim3(kTileThreads), 0, stream,
                       keys, n, w.tu_keys, w.tu_count, w.local);
    hipLaunchKernelGGL(k_dedup_global, dim3(grid_for(ntiles, 1, 1 << 16)), dim3(kGlobalThreads), 0, stream,
                       w.tu_keys, w.tu_count, ntiles, w.set_keys, w.set_ids, (uint64_t)(w.cap - 1), w.tu_slot,
                       unique, (unsigned long long*)n_unique_dev, w.misc);
    hipLaunchKernelGGL(k_dedup_compose, dim3(grid_for(n, 256 * 4, 1 << 16)), dim3(256), 0, stream,
                       w.local, n, w.tu_slot, w.set_ids, w.misc, inverse);
    return check_launch("dedup_unique_inverse");
}

}  // extern "C"
