// Bucket-walk helpers of the dynamic table, shared by the find-or-insert,
// erase, import and rehash kernels (internal header).
//
// MTGenRec (arXiv 2505.12663) Theorem 1: in a table of 2^n slots the walk
// h_t = h_0 + t*S mod 2^n visits every slot iff S is odd.  Here the walk is
// over buckets of min(16, M) slots (one 128-byte line of keys), so every
// bucket, hence every slot, is on each key's walk.
#pragma once

#include "htl_common.h"

namespace htl {

constexpr int kProbeBlock = 256;

// Lanes per key in the probe kernels (1, 2, 4, 8 or 16; default 2); the
// environment variable HTL_PROBE_LANES overrides it.
int probe_lanes();

// The G-bit slice of a wave ballot that belongs to this lane's group.
template <int G>
__device__ __forceinline__ uint32_t group_bits(uint64_t ballot, int gshift) {
    return (uint32_t)(ballot >> gshift) & ((1u << G) - 1u);
}

__device__ __forceinline__ int64_t clamp_count(int64_t n_max, const int64_t* n_dev) {
    if (!n_dev) return n_max;
    int64_t c = *n_dev;
    return c < 0 ? 0 : (c < n_max ? c : n_max);
}

// Writes the closed-form initial row of `key` into `slot` (the G lanes of a
// group cooperate) and zeroes its Adam moments.
template <int G>
__device__ void write_initial_row(const TableDev& T, int64_t slot, int64_t key, int gl) {
    const uint64_t base = row_base(key, T.init_base);
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    if ((row_bytes & 15) == 0) {
        const int vpr = (int)(row_bytes >> 4);
        u32x4* dst = reinterpret_cast<u32x4*>(T.rows) + slot * vpr;
        for (int v = gl; v < vpr; v += G) __builtin_nontemporal_store(init_vec(base, v, T.dtype), dst + v);
    } else if (T.dtype == HTL_F32) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(T.rows) + slot * T.dim;
        for (int j = gl; j < T.dim; j += G) dst[j] = init_elem_bits(base, j, T.dtype);
    } else {
        uint16_t* dst = reinterpret_cast<uint16_t*>(T.rows) + slot * T.dim;
        for (int j = gl; j < T.dim; j += G) dst[j] = (uint16_t)init_elem_bits(base, j, T.dtype);
    }
    if (T.m) {
        for (int j = gl; j < T.dim; j += G) {
            T.m[slot * T.dim + j] = 0.0f;
            T.v[slot * T.dim + j] = 0.0f;
        }
    }
}

// Writes the initial rows (and zeroed Adam moments) of every key that the
// groups of this wave have just inserted, with all 64 lanes: each 16-byte
// vector of those rows is one lane's store, so the stores of a row leave
// together and no lane of a group that found its key sits idle.  The stores
// are non-temporal: nothing in this kernel reads the rows again, and kept
// out of L2 they are not written back while the next kernels run (the
// large-table step 0.627 -> 0.610 ms, its gather 0.304 -> 0.289 ms; the
// merged-tables step 2.847 -> 2.775 ms).  Must be
// called by the whole wave; `ins` marks a group that inserted key `k` at
// `slot` (every lane of the group passes the same values).  Needs 16-byte
// rows (dim*elem_bytes % 16 == 0).
template <int G>
__device__ void write_initial_rows_wave(const TableDev& T, bool ins, int64_t slot, int64_t k) {
    const int lane = lane_id();
    const bool lead = ins && (lane & (G - 1)) == 0;
    const uint64_t lm = __ballot(lead);
    const int cnt = __popcll(lm);
    if (cnt == 0) return;
    // Forward-permute the leaders' (slot, row seed) to lanes 0..cnt-1 (the
    // other lanes fill lanes cnt..63, so every destination is written once).
    const uint64_t below = lanemask_lt();
    const int dst = lead ? __popcll(lm & below) : cnt + __popcll(~lm & below);
    const uint64_t seed = row_base(k, T.init_base);
    const int s_c = __builtin_amdgcn_ds_permute(dst * 4, (int)slot);
    const int lo_c = __builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)seed);
    const int hi_c = __builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)(seed >> 32));
    const int vpr = (T.dim * T.elem_bytes) >> 4;
    const int mvv = T.m ? (T.dim >> 2) : 0;       // 16-byte vectors per moment row
    const int per = vpr + 2 * mvv;
    const int total = cnt * per;
    u32x4* rows = reinterpret_cast<u32x4*>(T.rows);
    for (int b0 = 0; b0 < total; b0 += 64) {
        const int w = b0 + lane;
        int r = w / per;
        if (r >= cnt) r = cnt - 1;
        const int64_t s = (int64_t)(uint32_t)__shfl(s_c, r);
        const uint64_t base = ((uint64_t)(uint32_t)__shfl(hi_c, r) << 32) | (uint32_t)__shfl(lo_c, r);
        if (w < total) {
            const int u = w - r * per;
            if (u < vpr) {
                __builtin_nontemporal_store(init_vec(base, u, T.dtype), rows + s * vpr + u);
            } else {
                const u32x4 z = {0u, 0u, 0u, 0u};
                float* mv = (u < vpr + mvv) ? T.m : T.v;
                const int q = (u < vpr + mvv) ? u - vpr : u - vpr - mvv;
                __builtin_nontemporal_store(z, reinterpret_cast<u32x4*>(mv) + s * mvv + q);
            }
        }
    }
}

// One bucket as seen by a group of G lanes: lane gl holds the SPL = 16/G
// consecutive slots [gl*SPL, gl*SPL + SPL), read with 16-byte loads when the
// bucket is a full 16 slots.  Slots outside [from, W) are not examined.
// Returns, as bucket-relative slot numbers (-1 for none), the first slot
// holding `k` and the first free slot, and whether the bucket holds an EMPTY
// slot; *free_val receives the content of that first free slot.
typedef int64_t i64x2 __attribute__((ext_vector_type(2)));

template <int G>
__device__ __forceinline__ void probe_bucket(const int64_t* bucket, int64_t k, int gl, int gshift, int from, int W,
                                             int& hit, int& free_slot, int64_t& free_val, bool& has_empty) {
    constexpr int SPL = 16 / G;
    int64_t v[SPL];
    const int s0 = gl * SPL;
    if (W == 16 && SPL >= 2) {
#pragma unroll
        for (int q = 0; q < SPL / 2; ++q) {
            const i64x2 x = *reinterpret_cast<const i64x2*>(bucket + s0 + 2 * q);
            v[2 * q] = x.x;
            v[2 * q + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) v[j] = (s0 + j < W) ? peek_key(bucket + s0 + j) : kEmpty;
    }
    int mj = SPL, fj = SPL;
    bool emp = false;
#pragma unroll
    for (int j = SPL - 1; j >= 0; --j) {
        const int s = s0 + j;
        if (s >= from && s < W) {
            if (v[j] == k) mj = j;
            if (v[j] == kEmpty || v[j] == kTomb) fj = j;
            if (v[j] == kEmpty) emp = true;
        }
    }
    hit = -1;
    free_slot = -1;
    free_val = 0;
    const uint32_t mb = group_bits<G>(__ballot(mj < SPL), gshift);
    if (mb) {
        const int l = __builtin_ctz(mb);
        hit = l * SPL + __shfl(mj, gshift + l);
    }
    const uint32_t fb = group_bits<G>(__ballot(fj < SPL), gshift);
    if (fb) {
        const int l = __builtin_ctz(fb);
        int64_t fv = 0;
#pragma unroll
        for (int j = 0; j < SPL; ++j)
            if (j == fj) fv = v[j];
        const int fjl = __shfl(fj, gshift + l);
        free_slot = l * SPL + fjl;
        free_val = __shfl(fv, gshift + l);
    }
    has_empty = group_bits<G>(__ballot(emp), gshift) != 0;
}

// Walks the table for key k with the G lanes of this group, without
// inserting: returns the slot holding k, or -1 (the walk ends at the first
// bucket with an EMPTY slot, or after every bucket).
template <int G>
__device__ __forceinline__ int64_t find_key(const TableDev& T, int64_t k, int gl, int gshift) {
    if (k == kEmpty || k == kTomb) return -1;
    const int W = 1 << T.bucket_log2;
    const uint64_t nb = T.bucket_mask + 1;
    const uint64_t h = mix64((uint64_t)k ^ T.salt);
    const uint64_t S = ((h >> 32) | 1ull) & T.bucket_mask;
    uint64_t b = h & T.bucket_mask;
    for (uint64_t t = 0; t < nb; ++t) {
        const int64_t base = (int64_t)(b << T.bucket_log2);
        int hit, fs;
        int64_t fv;
        bool has_empty;
        probe_bucket<G>(T.keys + base, k, gl, gshift, 0, W, hit, fs, fv, has_empty);
        if (hit >= 0) return base + hit;
        if (has_empty) return -1;
        b = (b + S) & T.bucket_mask;
    }
    return -1;
}

// Walks the table for key k with the G lanes of this group and returns its
// status; *slot receives the slot (FOUND / INSERTED) or -1.  Inserts claim
// the first free slot of the walk with a 64-bit CAS (the caller writes the
// row); a lost CAS either reveals the key itself (FOUND) or another key, and
// the walk then resumes right after that slot.
template <int G>
__device__ __forceinline__ int find_or_insert_key(const TableDev& T, int64_t k, int gl, int gshift,
                                                  int64_t* slot_out) {
    const int W = 1 << T.bucket_log2;
    const uint64_t nb = T.bucket_mask + 1;
    int st = HT_FULL;
    int64_t slot = -1;
    if (k == kEmpty || k == kTomb) {
        *slot_out = -1;
        return HT_RESERVED;
    }
    const uint64_t h = mix64((uint64_t)k ^ T.salt);
    const uint64_t S = ((h >> 32) | 1ull) & T.bucket_mask;
    uint64_t b = h & T.bucket_mask;
    uint64_t t = 0;           // buckets walked so far
    int from = 0;             // first slot of bucket b still to examine
    int64_t ff = -1;          // first free slot seen on the walk
    int64_t ffv = 0;          // its content when seen (EMPTY or TOMBSTONE)
    uint64_t ff_b = 0, ff_t = 0;
    // Every pass of this loop either ends the walk or moves it forward by at
    // least one slot, so it runs at most M + M/16 times.
    for (int64_t guard = 0; guard <= T.capacity + (int64_t)nb; ++guard) {
        bool found = false;          // else: saw EMPTY, or walked every bucket
        while (t < nb) {
            const int64_t base = (int64_t)(b << T.bucket_log2);
            int hit, fs;
            int64_t fv;
            bool has_empty;
            probe_bucket<G>(T.keys + base, k, gl, gshift, from, W, hit, fs, fv, has_empty);
            if (hit >= 0) {
                slot = base + hit;
                found = true;
                break;
            }
            if (ff < 0 && fs >= 0) {
                ff = base + fs;
                ffv = fv;
                ff_b = b;
                ff_t = t;
            }
            if (has_empty) break;
            from = 0;
            b = (b + S) & T.bucket_mask;
            ++t;
        }
        if (found) {
            st = HT_FOUND;
            break;
        }
        if (ff < 0) {            // the whole walk -- every slot -- is taken
            st = HT_FULL;
            break;
        }
        int64_t old = 0;
        if (gl == 0) old = cas_key(T.keys + ff, ffv, k);
        old = __shfl(old, gshift);
        if (old == ffv) {
            slot = ff;
            st = HT_INSERTED;
            break;
        }
        if (old == k) {          // the same key was inserted concurrently
            slot = ff;
            st = HT_FOUND;
            break;
        }
        // Another key took the slot: resume the walk right after it.
        b = ff_b;
        t = ff_t;
        from = (int)(ff & (W - 1)) + 1;
        if (from >= W) {
            from = 0;
            b = (b + S) & T.bucket_mask;
            ++t;
        }
        ff = -1;
    }
    *slot_out = slot;
    return st;
}

}  // namespace htl
