// Internal definitions shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "htl.h"

namespace htl {

// ------------------------------------------------------------- errors ----
void set_error(const std::string& msg);
void clear_error();
htl_status fail(htl_status code, const std::string& msg);
htl_status check_launch(const char* what);   // hipGetLastError after enqueues

#define HTL_REQUIRE(cond, msg)                                   \
    do {                                                         \
        if (!(cond)) return ::htl::fail(HTL_ERR_INVALID, (msg)); \
    } while (0)

#define HTL_HIP(call)                                                                   \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess)                                                           \
            return ::htl::fail(HTL_ERR_DEVICE, std::string(#call ": ") + hipGetErrorString(e_)); \
    } while (0)

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// -------------------------------------------------------------- table ----
constexpr int64_t kEmpty = -1;       // HT_EMPTY_KEY
constexpr int64_t kTomb = -2;        // HT_TOMBSTONE_KEY
// last_seen of every slot that holds no live key (EMPTY, TOMBSTONE), so a
// pass over last_seen alone tells the live slots apart; steps stamped into
// last_seen are below it.
constexpr uint32_t kLsDead = 0xFFFFFFFFu;
constexpr int kBucketLog2 = 4;       // 16 slots = 128 bytes of keys per bucket

// Everything a kernel needs to know about a table, passed by value.
struct TableDev {
    int64_t* keys;
    void* rows;
    uint32_t* last_seen;   // nullable
    float* m;              // nullable
    float* v;              // nullable
    int64_t capacity;
    uint64_t bucket_mask;  // number of buckets - 1
    int bucket_log2;       // slots per bucket = 1 << bucket_log2 (<= 4)
    int dim;
    int elem_bytes;        // 4 (fp32) or 2 (bf16)
    int dtype;
    uint64_t init_base;    // mix64(init_seed)
    uint64_t salt;         // probe-hash salt
    int32_t* rowid;        // growable tables: row handle of each live slot; null: row = slot
};

// ------------------------------------------------------- access log ----
// A table created with HT_META_ACCESS_LOG records, at every find-or-insert,
// one 8-byte entry per key it is given: (slot, step) when the call inserts
// the key or moves its last_seen to `step`, else kLogNoSlot.  Entries go to
// a ring in call order, so along the ring the steps never decrease.  Beside
// the ring, one record per step (indexed by step mod kLogSteps) keeps where
// the step's entries lie and how many live keys have last_seen == step:
// each stamp adds one to its step and takes one from the key's previous
// step, each erase takes one from the erased key's step.  An entry is
// current iff last_seen[slot] still equals its step; the current entries of
// steps <= s are exactly the live keys with last_seen <= s (a key gets one
// entry per step it is stamped in).  The eviction choice reads the step
// counts to find the cut step, then only the ring entries up to that
// step's end, instead of last_seen of every slot.
// A step's count is kept as kLogSubs partial counts, each on a cache line of
// its own, that the blocks of a call add to by block index: thousands of
// blocks adding to one line serialise in the L2 (on the online workload,
// find-or-insert went 63 -> 181 us and erase 14 -> 92 us with one count
// per step).
constexpr int kLogStepsLog2 = 12;
constexpr int64_t kLogSteps = (int64_t)1 << kLogStepsLog2;
constexpr uint32_t kLogStepMask = (uint32_t)kLogSteps - 1u;
constexpr uint32_t kLogNoSlot = 0xFFFFFFFFu;
constexpr int kLogBins = 256;        // per-block LDS sums of steps left / erased
constexpr int kLogSubs = 32;         // partial counts per step
constexpr int kLogCntStride = 16;    // int64 words between partial counts (128 bytes)

struct LogSeg {
    uint32_t step;        // the step this record belongs to (0xFFFFFFFF: none yet)
    uint32_t pad;
    uint64_t begin, end;  // ring positions of the step's entries (unwrapped)
};

struct LogState {
    uint64_t head[2];     // next ring position, double-buffered by call parity
    uint64_t tail;        // no current entry lies before it
    uint32_t s_min;       // no live key has last_seen below it
    int32_t bad;          // set once the log stopped covering every live key
};

struct LogDev {
    uint64_t* entries;    // [cap]: slot | step << 32
    LogSeg* segs;         // [kLogSteps]
    int64_t* cnt;         // [kLogSteps][kLogSubs][kLogCntStride]: live keys with last_seen == step,
                          // as kLogSubs partial sums (word 0 of each line)
    LogState* st;
    uint64_t cap_mask;    // cap - 1 (cap a power of two)
};

// Row-space index of a live slot.
__device__ __forceinline__ int64_t row_of(const TableDev& T, int64_t slot) {
    return T.rowid ? (int64_t)T.rowid[slot] : slot;
}

// A device array in a reserved virtual range that grows by mapping more
// physical memory at its end (growable tables' row space).
struct VmArray {
    void* base = nullptr;
    size_t reserved = 0;   // bytes of address space
    size_t mapped = 0;     // bytes mapped from base
    std::vector<hipMemGenericAllocationHandle_t> handles;
    std::vector<size_t> sizes;
};

// Row-handle bookkeeping of a growable table, and per-call temporaries of
// any table (device memory, allocated on first use).
struct RowAlloc {
    int64_t* state = nullptr;      // [0] next never-used row, [1] handles on the free stack
    int32_t* free_stack = nullptr; // [rows]
    int32_t* chunk_cnt = nullptr;  // per-call temporaries: per 64-key chunk counts ...
    int32_t* chunk_off = nullptr;  // ... their exclusive prefix ...
    int32_t* row_tmp = nullptr;    // ... a row handle per key (erase)
    uint8_t* status_tmp = nullptr; // ... and a status per key (erase without status)
    void* scan_tmp = nullptr;
    void* tmp_base = nullptr;      // one allocation holding the temporaries
    int64_t tmp_keys = 0;          // keys the temporaries are sized for
    // export temporaries: per 4096-slot chunk counts and their prefix
    int32_t* exp_cnt = nullptr;
    int32_t* exp_off = nullptr;
    void* exp_scan = nullptr;
    void* exp_base = nullptr;
    int64_t exp_chunks = 0;
};

}  // namespace htl

struct htl_table {
    int device;
    int capacity_log2;
    int dim;
    htl_dtype dtype;
    uint64_t init_seed;
    uint32_t flags;
    uint32_t max_step;   // largest step any find-or-insert stamped since create/clear
    htl::TableDev dev;
    int max_capacity_log2;
    htl::VmArray vm_rows, vm_m, vm_v;   // growable tables only
    htl::RowAlloc alloc;                // handles: growable only; temporaries: any table
    // access log (HT_META_ACCESS_LOG): device storage, and what the host
    // knows of it
    htl::LogDev log;
    bool log_ok;          // false once a call broke the log's premises
    bool log_first;       // no call logged since create / clear
    int log_par;          // parity of the next logged call
    bool erase_pending;   // an erase ran while max_step was erase_step
    uint32_t erase_step;
};

namespace htl {

// --------------------------------------------------------- device math ----
__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The closed-form initial row of a key, 16 bytes at a time.  Row words come
// in pairs from one SplitMix64 output: output c (0-based) of the stream
// seeded with base = mix64(key ^ mix64(seed)) is mix64(base + (c+1)*gamma);
// its high half is word 2c, its low half word 2c+1.
//   fp32 element j: ((word_j >> 8) - 2^23) * 2^-26
//   bf16 element j: ((word_j >> 24) - 128) * 2^-10
__device__ __forceinline__ uint64_t row_base(int64_t key, uint64_t init_base) {
    return mix64((uint64_t)key ^ init_base);
}
__device__ __forceinline__ uint64_t row_word_pair(uint64_t base, uint32_t c) {
    return mix64(base + (uint64_t)(c + 1) * kGamma);
}
__device__ __forceinline__ float init_f32(uint32_t w) {
    return (float)((int32_t)(w >> 8) - (1 << 23)) * 0x1p-26f;
}
__device__ __forceinline__ uint32_t init_bf16_bits(uint32_t w) {
    // exact: |q| <= 128 needs at most 8 significant bits
    return __float_as_uint((float)((int32_t)(w >> 24) - 128) * 0x1p-10f) >> 16;
}
// 16-byte vector v of the initial row (elements [v*E, v*E + E) with E = 4
// fp32 or 8 bf16).
// Consecutive outputs of the stream are seeded base + (c+1)*gamma, so the
// states of one vector's outputs differ by gamma and follow by addition
// (mod 2^64: the same values as one multiply each).
__device__ __forceinline__ u32x4 init_vec(uint64_t base, int v, int dtype) {
    u32x4 out;
    if (dtype == HTL_F32) {
        const uint64_t z0 = base + (uint64_t)(2 * v + 1) * kGamma;
        const uint64_t r0 = mix64(z0);
        const uint64_t r1 = mix64(z0 + kGamma);
        out.x = __float_as_uint(init_f32((uint32_t)(r0 >> 32)));
        out.y = __float_as_uint(init_f32((uint32_t)r0));
        out.z = __float_as_uint(init_f32((uint32_t)(r1 >> 32)));
        out.w = __float_as_uint(init_f32((uint32_t)r1));
    } else {
        uint32_t o[4];
        uint64_t z = base + (uint64_t)(4 * v + 1) * kGamma;
#pragma unroll
        for (int q = 0; q < 4; ++q, z += kGamma) {
            const uint64_t r = mix64(z);
            o[q] = init_bf16_bits((uint32_t)(r >> 32)) | (init_bf16_bits((uint32_t)r) << 16);
        }
        out.x = o[0]; out.y = o[1]; out.z = o[2]; out.w = o[3];
    }
    return out;
}
// Element j of the initial row as raw bits (fp32 bits, or bf16 bits in the
// low half) -- for rows whose byte length is not a multiple of 16.
__device__ __forceinline__ uint32_t init_elem_bits(uint64_t base, int j, int dtype) {
    uint64_t r = row_word_pair(base, (uint32_t)(j >> 1));
    uint32_t w = (j & 1) ? (uint32_t)r : (uint32_t)(r >> 32);
    return dtype == HTL_F32 ? __float_as_uint(init_f32(w)) : init_bf16_bits(w);
}

// ------------------------------------------------------ wave helpers ----
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Cacheable single-copy-atomic load of a key slot that other workgroups may
// CAS during the same kernel.  It may return an older value of the slot.
// Within one kernel a slot only ever goes from free (EMPTY or TOMBSTONE) to a
// key -- never back -- so an old value can only show a slot as free that is
// already taken; every claim goes through a CAS whose returned value is the
// slot's true content, and the probe loops act on that value.  Between
// kernels the runtime's acquire/release makes every write visible.
__device__ __forceinline__ int64_t peek_key(const int64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint64_t peek_u64(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ int64_t cas_key(int64_t* p, int64_t expected, int64_t desired) {
    return (int64_t)atomicCAS((unsigned long long*)p, (unsigned long long)expected,
                              (unsigned long long)desired);
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch-size helper: blocks for `items` work items of `per_block` each,
// clamped to [1, cap] (kernels loop grid-stride beyond the cap).
inline unsigned grid_for(int64_t items, int64_t per_block, int64_t cap = (1 << 20)) {
    int64_t b = ceil_div(items, per_block);
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (unsigned)b;
}

}  // namespace htl
