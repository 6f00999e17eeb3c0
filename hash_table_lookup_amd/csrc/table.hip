// Dynamic open-addressing embedding table: create/clear/destroy,
// find-or-insert, erase, compact scan.
//
// MTGenRec (arXiv 2505.12663): Abstract and Figure 5 (a hash-based dynamic
// embedding table replaces static tables so embeddings can be inserted and
// deleted in real time), Theorem 1 (in a table of 2^n slots the walk
// h_t = h_0 + t*S mod 2^n visits every slot iff S is odd).  MTGR (arXiv
// 2505.18654) section 5, "Embedding Management": keys map to embedding
// vectors plus metadata, and live keys can be scanned compactly.
//
// Layout in HBM: keys int64[M] (EMPTY = -1, TOMBSTONE = -2), rows
// dtype[M][dim] indexed by slot, optional last_seen uint32[M], optional Adam
// moments float[M][dim].
//
// Probing (this library's layout, not the pages'): the M slots form
// min(16, M)-slot buckets, one 128-byte line of keys each.  A key's walk
// visits bucket b_t = b_0 + t*S mod (M/16) with S odd, so by Theorem 1 over the
// buckets every bucket -- hence every slot -- is on the walk.  Within a bucket
// the slots are taken in order.  A group of G lanes (1, 2, 4, 8 or 16) works
// on one key, each lane holding 16/G consecutive slots of the bucket, so a
// wavefront keeps 64/G keys in flight; the group loads the bucket's 128-byte line together and
// ballots decide found / first free slot / EMPTY seen.  An insert claims the
// first free (EMPTY or TOMBSTONE) slot of the walk with a 64-bit CAS; if the
// CAS loses, the returned key is either the key itself (FOUND) or another
// key, and the walk resumes right after that slot.
#include <cstdlib>

#include "probe.h"

namespace htl {

namespace {
thread_local std::string g_last_error;
constexpr uint64_t kProbeSalt = 0x2545F4914F6CDD1Dull;
}  // namespace

int probe_lanes() {
    static int lanes = [] {
        const char* e = getenv("HTL_PROBE_LANES");
        int v = e ? atoi(e) : 4;
        return (v == 1 || v == 2 || v == 4 || v == 8 || v == 16) ? v : 4;
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

template <int G>
__global__ __launch_bounds__(kProbeBlock) void k_find_or_insert(
    TableDev T, const int64_t* __restrict__ keys, int64_t n_max, const int64_t* __restrict__ n_dev,
    uint32_t step, int32_t* __restrict__ slots, uint8_t* __restrict__ status) {
    const int64_t n = clamp_count(n_max, n_dev);
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int64_t group0 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / G;
    const int64_t ngroups = (int64_t)gridDim.x * blockDim.x / G;

    for (int64_t i = group0; i < n; i += ngroups) {
        const int64_t k = keys[i];
        int64_t slot;
        const int st = find_or_insert_key<G>(T, k, gl, gshift, &slot);
        if (st == HT_INSERTED) write_initial_row<G>(T, slot, k, gl);
        if (gl == 0) {
            if ((st == HT_FOUND || st == HT_INSERTED) && T.last_seen) T.last_seen[slot] = step;
            slots[i] = (int32_t)slot;
            status[i] = (uint8_t)st;
        }
    }
}

template <int G>
__global__ __launch_bounds__(kProbeBlock) void k_erase(TableDev T, const int64_t* __restrict__ keys,
                                                       int64_t n, uint8_t* __restrict__ status) {
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
                    break;
                }
                if (has_empty) break;
                b = (b + S) & T.bucket_mask;
            }
        }
        if (gl == 0 && status) status[i] = (uint8_t)st;
    }
}

// Compact scan of live slots.  Each block owns a contiguous range of
// kScanPerBlock slots, counts its live slots, reserves an output range with
// one atomic, and writes them there (thread-major order within the block).
constexpr int kScanBlock = 256;
constexpr int kScanPerThread = 16;
constexpr int kScanPerBlock = kScanBlock * kScanPerThread;

__global__ void k_zero_i64(int64_t* p) { *p = 0; }

__global__ __launch_bounds__(kScanBlock) void k_scan_live(TableDev T, int64_t* __restrict__ out_keys,
                                                         uint32_t* __restrict__ out_ls,
                                                         int32_t* __restrict__ out_slots,
                                                         unsigned long long* __restrict__ counter) {
    __shared__ int s_warp[kScanBlock / 64];
    __shared__ unsigned long long s_base;
    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    for (int64_t blk = blockIdx.x; blk * kScanPerBlock < T.capacity; blk += gridDim.x) {
        const int64_t start = blk * kScanPerBlock;
        int64_t k[kScanPerThread];
        uint32_t live = 0;
#pragma unroll
        for (int j = 0; j < kScanPerThread; ++j) {
            const int64_t s = start + (int64_t)j * kScanBlock + tid;
            k[j] = s < T.capacity ? T.keys[s] : kEmpty;
            if (k[j] != kEmpty && k[j] != kTomb) live |= 1u << j;
        }
        // per-wave counts of each round j, then a block-wide exclusive prefix
        int my_total = __popc(live);
        int incl = my_total;
        for (int off = 1; off < 64; off <<= 1) {
            int y = __shfl_up(incl, off);
            if (lane_id() >= off) incl += y;
        }
        if (lane_id() == 63) s_warp[wid] = incl;
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int w = 0; w < kScanBlock / 64; ++w) {
                int c = s_warp[w];
                s_warp[w] = run;
                run += c;
            }
            s_base = run ? atomicAdd(counter, (unsigned long long)run) : 0ull;
        }
        __syncthreads();
        int64_t pos = (int64_t)s_base + s_warp[wid] + (incl - my_total);
#pragma unroll
        for (int j = 0; j < kScanPerThread; ++j) {
            if (live & (1u << j)) {
                const int64_t s = start + (int64_t)j * kScanBlock + tid;
                if (out_keys) out_keys[pos] = k[j];
                if (out_ls) out_ls[pos] = T.last_seen ? T.last_seen[s] : 0u;
                if (out_slots) out_slots[pos] = (int32_t)s;
                ++pos;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ host side --
htl_status fill_keys_empty(const TableDev& T, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_i64, dim3(grid_for(T.capacity, 256 * 8, 1 << 16)), dim3(256), 0, s,
                       T.keys, T.capacity, kEmpty);
    return check_launch("clear table keys");
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
    HTL_REQUIRE((flags & ~(uint32_t)(HT_META_LAST_SEEN | HT_ADAM_STATE)) == 0, "ht_create: unknown flag");
    HTL_REQUIRE(!(flags & HT_ADAM_STATE) || dtype == HTL_F32, "ht_create: Adam state needs an fp32 table");

    htl_table* t = new htl_table();
    t->capacity_log2 = capacity_log2;
    t->dim = dim;
    t->dtype = dtype;
    t->init_seed = init_seed;
    t->flags = flags;
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
        if (T.keys) (void)hipFree(T.keys);
        if (T.rows) (void)hipFree(T.rows);
        if (T.last_seen) (void)hipFree(T.last_seen);
        if (T.m) (void)hipFree(T.m);
        if (T.v) (void)hipFree(T.v);
        delete t;
    };
    const size_t M = (size_t)T.capacity;
    const size_t row_bytes = M * (size_t)dim * (size_t)T.elem_bytes;
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
    if (st == HTL_OK && T.last_seen) {
        hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(T.capacity, 256 * 8, 1 << 16)), dim3(256), 0,
                           stream, T.last_seen, T.capacity, 0u);
        st = check_launch("clear last_seen");
    }
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
    (void)hipFree(T.keys);
    (void)hipFree(T.rows);
    if (T.last_seen) (void)hipFree(T.last_seen);
    if (T.m) (void)hipFree(T.m);
    if (T.v) (void)hipFree(T.v);
    delete t;
    HTL_HIP(hipSetDevice(cur));
    return HTL_OK;
}

htl_status ht_clear(htl_table* t, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_clear: null table");
    t->max_step = 0u;
    return fill_keys_empty(t->dev, stream);
}

htl_status ht_find_or_insert(htl_table* t, const int64_t* keys, int64_t n_max, const int64_t* n_dev,
                             uint32_t step, int32_t* slots, uint8_t* status, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_find_or_insert: null table");
    HTL_REQUIRE(n_max >= 0 && n_max < ((int64_t)1 << 31), "ht_find_or_insert: n_max out of range");
    if (n_max == 0) return HTL_OK;
    HTL_REQUIRE(keys && slots && status, "ht_find_or_insert: null keys/slots/status");
    HTL_REQUIRE(aligned(keys, 8) && aligned(slots, 4) && (!n_dev || aligned(n_dev, 8)),
                "ht_find_or_insert: misaligned pointer");
    if (step > t->max_step) t->max_step = step;
    const int G = probe_lanes();
    const unsigned grid = grid_for(n_max, kProbeBlock / G);
#define HTL_FOI(GG)                                                                                        \
    hipLaunchKernelGGL(k_find_or_insert<GG>, dim3(grid), dim3(kProbeBlock), 0, stream, t->dev, keys, n_max, \
                       n_dev, step, slots, status)
    switch (G) {
        case 1: HTL_FOI(1); break;
        case 2: HTL_FOI(2); break;
        case 8: HTL_FOI(8); break;
        case 16: HTL_FOI(16); break;
        default: HTL_FOI(4); break;
    }
#undef HTL_FOI
    return check_launch("ht_find_or_insert");
}

htl_status ht_erase(htl_table* t, const int64_t* keys, int64_t n, uint8_t* status, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_erase: null table");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "ht_erase: n out of range");
    if (n == 0) return HTL_OK;
    HTL_REQUIRE(keys && aligned(keys, 8), "ht_erase: null or misaligned keys");
    hipLaunchKernelGGL(k_erase<8>, dim3(grid_for(n, kProbeBlock / 8)), dim3(kProbeBlock), 0, stream, t->dev, keys,
                       n, status);
    return check_launch("ht_erase");
}

htl_status ht_scan(const htl_table* t, int64_t* keys, uint32_t* last_seen, int32_t* slots,
                   int64_t* n_live_dev, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_scan: null table");
    HTL_REQUIRE(n_live_dev && aligned(n_live_dev, 8), "ht_scan: null or misaligned n_live_dev");
    HTL_REQUIRE(!keys || aligned(keys, 8), "ht_scan: misaligned keys");
    hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(1), 0, stream, n_live_dev);
    hipLaunchKernelGGL(k_scan_live, dim3(grid_for(t->dev.capacity, kScanPerBlock, 1 << 16)),
                       dim3(kScanBlock), 0, stream, t->dev, keys, last_seen, slots,
                       (unsigned long long*)n_live_dev);
    return check_launch("ht_scan");
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
    return HTL_OK;
}

}  // extern "C"
