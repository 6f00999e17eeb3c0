// Device-side invariant checks of a build with -DHTL_DEBUG.
//
// After each call that changes or derives table state, a debug build
// launches a check kernel on the same stream.  A check records what it finds
// wrong as bits in a per-device flag word (vector atomics; nothing traps or
// stops a kernel); htl_debug_flags reads and clears the word.  Release builds
// compile the same helpers as empty functions.
//   find-or-insert: a FOUND or INSERTED key sits in the slot returned (fixed
//     tables), and walking its buckets from its first one it occurs exactly
//     once before a bucket with an EMPTY slot, within M/16 buckets (every
//     bucket once: Theorem 1 of MTGenRec at bucket level bounds the walk);
//     a FULL key has no free slot and no copy anywhere on its walk;
//   dedup: unique[inverse[i]] == keys[i] and inverse[i] < n_unique <= n;
//   access log: no live count of a step in [s_min, s_now] is negative.
#include "debug.h"

namespace htl {
namespace {

__device__ uint32_t g_debug_flags;   // one word per device

#ifdef HTL_DEBUG
__device__ __forceinline__ void flag(uint32_t* f, uint32_t bit) { atomicOr(f, bit); }

// One thread per key (a debug build favours plainness over speed).
__global__ void k_dbg_foi(TableDev T, const int64_t* __restrict__ keys, int64_t n_max, const int64_t* __restrict__ n_dev,
                          const int32_t* __restrict__ slots, const uint8_t* __restrict__ status, uint32_t* f) {
    const int64_t n = n_dev ? (*n_dev < n_max ? *n_dev : n_max) : n_max;
    const int W = 1 << T.bucket_log2;
    const uint64_t nb = T.bucket_mask + 1;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int st = status[i];
        const int64_t k = keys[i];
        if (st != HT_FOUND && st != HT_INSERTED && st != HT_FULL) continue;
        if (st != HT_FULL && !T.rowid) {
            const int32_t s = slots[i];
            if (s < 0 || s >= T.capacity || T.keys[s] != k) flag(f, HTL_DEBUG_SLOT);
        }
        const uint64_t h = mix64((uint64_t)k ^ T.salt);
        const uint64_t S = ((h >> 32) | 1ull) & T.bucket_mask;
        uint64_t b = h & T.bucket_mask;
        int copies = 0;
        bool free_seen = false, ended = false;
        uint64_t t = 0;
        for (; t < nb; ++t) {
            const int64_t* kb = T.keys + (int64_t)(b << T.bucket_log2);
            bool empty = false;
            for (int j = 0; j < W; ++j) {
                const int64_t v = kb[j];
                copies += v == k;
                empty |= v == kEmpty;
                free_seen |= v == kEmpty || v == kTomb;
            }
            if (empty) {
                ended = true;
                break;
            }
            b = (b + S) & T.bucket_mask;
        }
        if (t > nb) flag(f, HTL_DEBUG_WALK);
        if (st == HT_FULL) {
            if (free_seen || copies != 0 || ended) flag(f, HTL_DEBUG_FULL);
        } else if (copies != 1) {
            flag(f, HTL_DEBUG_DUP);
        }
    }
}

__global__ void k_dbg_dedup(const int64_t* __restrict__ keys, int64_t n, const int64_t* __restrict__ unique,
                            const int32_t* __restrict__ inverse, const int64_t* __restrict__ n_unique, uint32_t* f) {
    const int64_t U = *n_unique;
    if (blockIdx.x == 0 && threadIdx.x == 0 && (U < 0 || U > n || (n > 0 && U == 0))) flag(f, HTL_DEBUG_DEDUP);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t u = inverse[i];
        if (u < 0 || u >= U || unique[u] != keys[i]) flag(f, HTL_DEBUG_DEDUP);
    }
}

__global__ void k_dbg_log(LogDev L, uint32_t s_now, uint32_t* f) {
    const uint32_t s0 = L.st->s_min;
    if (L.st->bad || s_now < s0 || (int64_t)(s_now - s0) >= kLogSteps) return;   // the log is not serving
    for (uint32_t s = s0 + threadIdx.x; s - s0 <= s_now - s0; s += blockDim.x) {
        if (L.segs[s & kLogStepMask].step != s) continue;
        const int64_t* c = L.cnt + (int64_t)(s & kLogStepMask) * kLogSubs * kLogCntStride;
        int64_t sum = 0;
        for (int q = 0; q < kLogSubs; ++q) sum += c[q * kLogCntStride];
        if (sum < 0) flag(f, HTL_DEBUG_LOG);
    }
}
#endif

// The device's flag word (its address is per device; taken once each).
uint32_t* flags_address() {
    static std::mutex mu;
    static std::vector<uint32_t*> addr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_flags)) != hipSuccess) return nullptr;
        addr[dev] = (uint32_t*)p;
    }
    return addr[dev];
}

}  // namespace

void debug_check_foi(const TableDev& T, const int64_t* keys, int64_t n_max, const int64_t* n_dev,
                     const int32_t* slots, const uint8_t* status, hipStream_t stream) {
#ifdef HTL_DEBUG
    if (n_max <= 0) return;
    uint32_t* f = flags_address();
    if (f)
        hipLaunchKernelGGL(k_dbg_foi, dim3(grid_for(n_max, 256, 4096)), dim3(256), 0, stream, T, keys, n_max, n_dev,
                           slots, status, f);
#else
    (void)T, (void)keys, (void)n_max, (void)n_dev, (void)slots, (void)status, (void)stream;
#endif
}

void debug_check_dedup(const int64_t* keys, int64_t n, const int64_t* unique, const int32_t* inverse,
                       const int64_t* n_unique_dev, hipStream_t stream) {
#ifdef HTL_DEBUG
    if (n <= 0) return;
    uint32_t* f = flags_address();
    if (f)
        hipLaunchKernelGGL(k_dbg_dedup, dim3(grid_for(n, 256, 4096)), dim3(256), 0, stream, keys, n, unique, inverse,
                           n_unique_dev, f);
#else
    (void)keys, (void)n, (void)unique, (void)inverse, (void)n_unique_dev, (void)stream;
#endif
}

void debug_check_log(const htl_table* t, hipStream_t stream) {
#ifdef HTL_DEBUG
    if (!t->log.entries || !t->log_ok) return;
    uint32_t* f = flags_address();
    if (f) hipLaunchKernelGGL(k_dbg_log, dim3(1), dim3(256), 0, stream, t->log, t->max_step, f);
#else
    (void)t, (void)stream;
#endif
}

}  // namespace htl

using namespace htl;

extern "C" {

int htl_debug_build(void) {
#ifdef HTL_DEBUG
    return 1;
#else
    return 0;
#endif
}

htl_status htl_debug_flags(uint32_t* flags_out) {
    clear_error();
    HTL_REQUIRE(flags_out != nullptr, "htl_debug_flags: null output");
    *flags_out = 0u;
    uint32_t* f = flags_address();
    if (!f) return fail(HTL_ERR_DEVICE, "htl_debug_flags: no address for the flag word");
    HTL_HIP(hipDeviceSynchronize());
    HTL_HIP(hipMemcpy(flags_out, f, sizeof(uint32_t), hipMemcpyDeviceToHost));
    HTL_HIP(hipMemset(f, 0, sizeof(uint32_t)));
    HTL_HIP(hipDeviceSynchronize());
    return HTL_OK;
}

}  // extern "C"
