// Eviction choice for an online table: the floor(live * num / den) live keys
// that are smallest by (last_seen, key).
//
// MTGenRec (arXiv 2505.12663), Abstract: embeddings are inserted and deleted
// in real time; MTGR (arXiv 2505.18654) section 5, "Embedding Management":
// every key carries metadata and live keys can be scanned compactly.  The
// pages name no eviction policy; least recently used, ties broken by the key
// value, is this library's.
//
// Steps, all on the device (no host synchronisation):
//   collect  -- compact the live slots' (last_seen, key) into candidate lists
//               and take the maximum last_seen;
//   select   -- radix select with 8-bit digits: per digit, LDS histograms of
//               the candidates that match the digits chosen so far, summed
//               into one 256-bin histogram, and one block picks the bucket
//               that holds the k-th smallest.  last_seen digits go first
//               (only as many as its maximum needs), then the 64-bit keys
//               (sign bit flipped so unsigned order is signed order), the
//               latter over the compacted list of candidates that tie on
//               last_seen;
//   emit     -- every candidate at or below the selected (last_seen, key)
//               is a victim.
#include "htl_common.h"

namespace htl {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;

struct LruState {
    unsigned long long n_live;
    unsigned long long n_ties;
    unsigned long long n_out;
    int64_t k;            // victims wanted
    int64_t k_rem;        // rank (1-based) still to find inside the current prefix
    uint32_t ls_max;
    uint32_t ls_digits;   // last_seen digits in use
    uint32_t ls_prefix;   // selected last_seen (complete after the last digit)
    uint32_t pad;
    uint64_t key_prefix;  // selected biased key
    uint32_t hist[256];
};

struct LruWs {
    LruState* st;
    uint32_t* cand_ls;    // [M]
    uint64_t* cand_key;   // [M], biased keys
    uint64_t* ties;       // [M]
    size_t bytes;
};

LruWs lru_layout(int64_t M, char* base) {
    LruWs w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.st = (LruState*)take(sizeof(LruState));
    w.cand_ls = (uint32_t*)take((size_t)M * 4);
    w.cand_key = (uint64_t*)take((size_t)M * 8);
    w.ties = (uint64_t*)take((size_t)M * 8);
    w.bytes = off;
    return w;
}

__device__ __forceinline__ uint64_t bias(int64_t k) { return (uint64_t)k ^ 0x8000000000000000ull; }

__global__ void k_lru_reset(LruState* st) {
    if (threadIdx.x == 0) {
        st->n_live = st->n_ties = st->n_out = 0ull;
        st->ls_max = 0u;
        st->ls_prefix = 0u;
        st->key_prefix = 0ull;
    }
    st->hist[threadIdx.x] = 0u;
}

// Compaction of live slots (block-level counting, one atomic per block).
__global__ __launch_bounds__(kThreads) void k_lru_collect(TableDev T, LruState* __restrict__ st,
                                                         uint32_t* __restrict__ cand_ls,
                                                         uint64_t* __restrict__ cand_key) {
    __shared__ int s_warp[kThreads / 64];
    __shared__ unsigned long long s_base;
    const int tid = threadIdx.x, wid = tid >> 6, lane = lane_id();
    constexpr int kPerBlock = kThreads * kPerThread;
    uint32_t my_max = 0;
    for (int64_t blk = blockIdx.x; blk * kPerBlock < T.capacity; blk += gridDim.x) {
        const int64_t start = blk * kPerBlock;
        int64_t k[kPerThread];
        uint32_t live = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t s = start + (int64_t)j * kThreads + tid;
            k[j] = s < T.capacity ? T.keys[s] : kEmpty;
            if (k[j] != kEmpty && k[j] != kTomb) live |= 1u << j;
        }
        const int mine = __popc(live);
        int incl = mine;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == 63) s_warp[wid] = incl;
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int w = 0; w < kThreads / 64; ++w) {
                const int c = s_warp[w];
                s_warp[w] = run;
                run += c;
            }
            s_base = run ? atomicAdd(&st->n_live, (unsigned long long)run) : 0ull;
        }
        __syncthreads();
        int64_t pos = (int64_t)s_base + s_warp[wid] + (incl - mine);
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            if (live & (1u << j)) {
                const int64_t s = start + (int64_t)j * kThreads + tid;
                const uint32_t ls = T.last_seen[s];
                my_max = ls > my_max ? ls : my_max;
                cand_ls[pos] = ls;
                cand_key[pos] = bias(k[j]);
                ++pos;
            }
        }
        __syncthreads();
    }
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t y = __shfl_xor(my_max, off);
        my_max = y > my_max ? y : my_max;
    }
    if (lane == 0 && my_max) atomicMax(&st->ls_max, my_max);
}

__global__ void k_lru_init(LruState* st, int64_t num, int64_t den) {
    const int64_t L = (int64_t)st->n_live;
    st->k = (L * num) / den;
    st->k_rem = st->k;
    uint32_t d = 1;
    while (d < 4 && (st->ls_max >> (8 * d)) != 0u) ++d;
    st->ls_digits = d;
}

// Histogram of last_seen digit `d` over candidates matching the higher digits.
__global__ __launch_bounds__(kThreads) void k_lru_hist_ls(LruState* __restrict__ st,
                                                         const uint32_t* __restrict__ cand_ls, int d) {
    if ((uint32_t)d >= st->ls_digits) return;
    __shared__ uint32_t s_h[256];
    s_h[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t L = (int64_t)st->n_live;
    const uint32_t hi_shift = 8u * (uint32_t)(d + 1);
    const uint32_t want = hi_shift >= 32 ? 0u : (st->ls_prefix >> hi_shift);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < L; i += stride) {
        const uint32_t x = cand_ls[i];
        const uint32_t hi = hi_shift >= 32 ? 0u : (x >> hi_shift);
        if (hi == want) atomicAdd(&s_h[(x >> (8 * d)) & 255u], 1u);
    }
    __syncthreads();
    if (s_h[threadIdx.x]) atomicAdd(&st->hist[threadIdx.x], s_h[threadIdx.x]);
}

// Histogram of key digit `d` over the tied candidates matching higher digits.
__global__ __launch_bounds__(kThreads) void k_lru_hist_key(LruState* __restrict__ st,
                                                          const uint64_t* __restrict__ ties, int d) {
    __shared__ uint32_t s_h[256];
    s_h[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t L = (int64_t)st->n_ties;
    const uint32_t hi_shift = 8u * (uint32_t)(d + 1);
    const uint64_t want = hi_shift >= 64 ? 0ull : (st->key_prefix >> hi_shift);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < L; i += stride) {
        const uint64_t x = ties[i];
        const uint64_t hi = hi_shift >= 64 ? 0ull : (x >> hi_shift);
        if (hi == want) atomicAdd(&s_h[(uint32_t)(x >> (8 * d)) & 255u], 1u);
    }
    __syncthreads();
    if (s_h[threadIdx.x]) atomicAdd(&st->hist[threadIdx.x], s_h[threadIdx.x]);
}

// One block of 256: pick the bucket holding rank k_rem, narrow the prefix,
// clear the histogram for the next digit.
__global__ __launch_bounds__(256) void k_lru_pick(LruState* st, int d, int is_key) {
    __shared__ uint32_t s_c[256];
    const int t = threadIdx.x;
    const bool active = is_key ? true : ((uint32_t)d < st->ls_digits);
    const uint32_t h = st->hist[t];
    s_c[t] = h;
    __syncthreads();
    if (t == 0 && active && st->k > 0) {
        int64_t rem = st->k_rem;
        int b = 0;
        for (; b < 255; ++b) {
            if ((int64_t)s_c[b] >= rem) break;
            rem -= s_c[b];
        }
        st->k_rem = rem;
        if (is_key) st->key_prefix |= (uint64_t)b << (8 * d);
        else st->ls_prefix |= (uint32_t)b << (8 * d);
    }
    __syncthreads();
    st->hist[t] = 0u;
}

__global__ __launch_bounds__(kThreads) void k_lru_ties(LruState* __restrict__ st,
                                                      const uint32_t* __restrict__ cand_ls,
                                                      const uint64_t* __restrict__ cand_key,
                                                      uint64_t* __restrict__ ties) {
    const int64_t L = (int64_t)st->n_live;
    if (st->k <= 0) return;
    const uint32_t thr = st->ls_prefix;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i0 = blockIdx.x * (int64_t)kThreads; i0 < L; i0 += stride) {
        const int64_t i = i0 + threadIdx.x;
        const bool tie = i < L && cand_ls[i] == thr;
        const uint64_t m = __ballot(tie);
        if (!m) continue;
        const int leader = __ffsll((unsigned long long)m) - 1;
        unsigned long long b = 0;
        if (lane_id() == leader) b = atomicAdd(&st->n_ties, (unsigned long long)__popcll(m));
        b = __shfl(b, leader);
        if (tie) ties[b + __popcll(m & lanemask_lt())] = cand_key[i];
    }
}

__global__ __launch_bounds__(kThreads) void k_lru_emit(LruState* __restrict__ st,
                                                      const uint32_t* __restrict__ cand_ls,
                                                      const uint64_t* __restrict__ cand_key,
                                                      int64_t* __restrict__ victims, int64_t cap,
                                                      int64_t* __restrict__ n_victims) {
    const int64_t L = (int64_t)st->n_live;
    const bool any = st->k > 0;
    const uint32_t thr = st->ls_prefix;
    const uint64_t kthr = st->key_prefix;
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_victims = st->k;
    if (!any) return;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i0 = blockIdx.x * (int64_t)kThreads; i0 < L; i0 += stride) {
        const int64_t i = i0 + threadIdx.x;
        bool v = false;
        uint64_t key = 0;
        if (i < L) {
            const uint32_t ls = cand_ls[i];
            key = cand_key[i];
            v = ls < thr || (ls == thr && key <= kthr);
        }
        const uint64_t m = __ballot(v);
        if (!m) continue;
        const int leader = __ffsll((unsigned long long)m) - 1;
        unsigned long long b = 0;
        if (lane_id() == leader) b = atomicAdd(&st->n_out, (unsigned long long)__popcll(m));
        b = __shfl(b, leader);
        const int64_t pos = (int64_t)b + __popcll(m & lanemask_lt());
        if (v && pos < cap) victims[pos] = (int64_t)(key ^ 0x8000000000000000ull);
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
    LruWs w = lru_layout(t->dev.capacity, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "ht_lru_select: workspace too small");
    const TableDev& T = t->dev;
    const unsigned gscan = grid_for(T.capacity, kThreads * kPerThread, 1 << 15);
    const unsigned gcand = grid_for(T.capacity, kThreads * 8, 1 << 14);
    hipLaunchKernelGGL(k_lru_reset, dim3(1), dim3(256), 0, stream, w.st);
    hipLaunchKernelGGL(k_lru_collect, dim3(gscan), dim3(kThreads), 0, stream, T, w.st, w.cand_ls, w.cand_key);
    hipLaunchKernelGGL(k_lru_init, dim3(1), dim3(1), 0, stream, w.st, num, den);
    for (int d = 3; d >= 0; --d) {
        hipLaunchKernelGGL(k_lru_hist_ls, dim3(gcand), dim3(kThreads), 0, stream, w.st, w.cand_ls, d);
        hipLaunchKernelGGL(k_lru_pick, dim3(1), dim3(256), 0, stream, w.st, d, 0);
    }
    hipLaunchKernelGGL(k_lru_ties, dim3(gcand), dim3(kThreads), 0, stream, w.st, w.cand_ls, w.cand_key, w.ties);
    for (int d = 7; d >= 0; --d) {
        hipLaunchKernelGGL(k_lru_hist_key, dim3(gcand), dim3(kThreads), 0, stream, w.st, w.ties, d);
        hipLaunchKernelGGL(k_lru_pick, dim3(1), dim3(256), 0, stream, w.st, d, 1);
    }
    hipLaunchKernelGGL(k_lru_emit, dim3(gcand), dim3(kThreads), 0, stream, w.st, w.cand_ls, w.cand_key, victims,
                       victims_cap, n_victims_dev);
    return check_launch("ht_lru_select");
}

}  // extern "C"
