// Fused forward lookup: dedup -> find-or-insert -> gather in one call, with
// the embedding table itself serving as the device-wide stage-2 set.
//
// MTGenRec (arXiv 2505.12663), TL;DR: a hash-based dynamic embedding table
// and two-stage ID deduplication for faster embedding lookups; MTGR (arXiv
// 2505.18654) section 5: IDs unique before and after the exchange, keys map
// to embedding vectors and metadata.
//
// The separate entry points dedup into a scratch set, then probe the table
// with the unique keys, then gather through slots[inverse[i]].  Every key of
// the batch ends up in the table anyway, so here the stage-1 tile survivors
// probe the table directly (find-or-insert, duplicates across tiles resolved
// by the walk itself) and mark the slot they land on in a byte map that the
// table keeps (all zero between calls).  Dense unique ids are ranks over that
// map -- one bit per slot, a prefix sum over 64-slot words -- so no atomic is
// spent on ids.  Unique keys come out in slot order.
//
//   k_dedup_tile          stage 1 in LDS (tile survivors, 16-bit local index)
//   k_lookup_claim<G>     survivors find-or-insert into the table; mark slot
//   k_lookup_spill_*      only if the table ran full: FULL keys get pseudo-
//                         slots in a spill set (one launch each, early exit)
//   k_lookup_words        map bytes -> 64-bit words + popcounts
//   prefix sum            word offsets (rank base per word)
//   k_lookup_emit         unique / slots / status per rank; re-zero the map
//   k_lookup_ids          per survivor: dense id (rank), INSERTED status
//   k_lookup_gather<TEAM> per ID: tile-local survivor record -> inverse + row
//
// Pseudo-slots: table slot p < M; key -1 -> M, key -2 -> M + 1 (RESERVED);
// FULL key in spill slot q -> 64 * words_table + q.
#include "probe.h"
#include "scan.h"
#include "tile_dedup.h"

namespace htl {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;

struct LookupWs {
    int64_t* tu_keys;      // [ntiles * kTile]
    int32_t* tu_count;     // [ntiles]
    uint16_t* local;       // [n]
    int32_t* tu_slot;      // [ntiles * kTile]: pseudo-slot of each survivor
    uint8_t* tu_ins;       // [ntiles * kTile]: 1 if this survivor inserted its key
    int32_t* tu_gid;       // [ntiles * kTile]: dense id of each survivor's key
    uint64_t* word_bits;   // [nwords]
    int32_t* word_cnt;     // [nwords]
    int32_t* word_off;     // [nwords + 1]
    void* scan_tmp;
    int64_t* spill_keys;   // [spill_cap]
    uint8_t* spill_map;    // [spill_cap]
    int32_t* flags;        // [0]: some survivor found the table full
    int64_t words_table, nwords;
    uint64_t spill_cap;
    size_t bytes;
};

LookupWs lookup_layout(int64_t M, int64_t n, char* base) {
    LookupWs w{};
    const int64_t ntiles = ceil_div(n, kTile);
    w.words_table = ceil_div(M + 2, 64);
    uint64_t cap = 64;
    while (cap < (uint64_t)(2 * n)) cap <<= 1;
    w.spill_cap = cap;
    w.nwords = w.words_table + (int64_t)(cap / 64);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.tu_keys = (int64_t*)take((size_t)ntiles * kTile * 8);
    w.tu_count = (int32_t*)take((size_t)ntiles * 4);
    w.local = (uint16_t*)take((size_t)n * 2);
    w.tu_slot = (int32_t*)take((size_t)ntiles * kTile * 4);
    w.tu_ins = (uint8_t*)take((size_t)ntiles * kTile);
    w.tu_gid = (int32_t*)take((size_t)ntiles * kTile * 4);
    w.word_bits = (uint64_t*)take((size_t)w.nwords * 8);
    w.word_cnt = (int32_t*)take((size_t)w.nwords * 4);
    w.word_off = (int32_t*)take((size_t)(w.nwords + 1) * 4);
    w.scan_tmp = take(scan_temp_bytes(w.nwords));
    w.spill_keys = (int64_t*)take(cap * 8);
    w.spill_map = (uint8_t*)take(cap);
    w.flags = (int32_t*)take(256);
    w.bytes = off;
    return w;
}

__device__ __forceinline__ u32x4 zero4() {
    u32x4 z;
    z.x = z.y = z.z = z.w = 0u;
    return z;
}

__global__ void k_lookup_reset(int32_t* flags) { flags[0] = 0; }
__global__ void k_write_zero_i64(int64_t* p) { *p = 0; }

// Survivors find-or-insert into the table, G lanes per survivor, over a flat
// grid of survivor positions (tile * kTile + j; positions past a tile's
// count are skipped).  The slot a survivor lands on is marked in the table's
// byte map (read first: a hot key's slot is written once, not once per tile).
template <int G>
__global__ __launch_bounds__(kBlock) void k_lookup_claim(TableDev T, const int64_t* __restrict__ tu_keys,
                                                        const int32_t* __restrict__ tu_count, int64_t npos,
                                                        uint32_t step, int32_t* __restrict__ tu_slot,
                                                        uint8_t* __restrict__ tu_ins, int32_t* __restrict__ flags) {
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int gshift = lane & ~(G - 1);
    const int64_t group0 = (blockIdx.x * (int64_t)kBlock + threadIdx.x) / G;
    const int64_t ngroups = (int64_t)gridDim.x * kBlock / G;
    for (int64_t pos = group0; pos < npos; pos += ngroups) {
        const int64_t tile = pos >> kTileLog2;
        const int j = (int)(pos & (kTile - 1));
        if (j >= tu_count[tile]) continue;
        const int64_t k = tu_keys[pos];
        int64_t p;
        int st;
        if (k == kEmpty) {
            p = T.capacity;
            st = HT_RESERVED;
        } else if (k == kTomb) {
            p = T.capacity + 1;
            st = HT_RESERVED;
        } else {
            int64_t slot;
            st = find_or_insert_key<G>(T, k, gl, gshift, &slot);
            if (st == HT_INSERTED) write_initial_row<G>(T, slot, k, gl);
            p = (st == HT_FULL) ? -1 : slot;
        }
        if (gl == 0) {
            if (p >= 0) {
                if (T.mark[p] == 0) T.mark[p] = 1;
                if (p < T.capacity && T.last_seen) T.last_seen[p] = step;
            } else {
                flags[0] = 1;
            }
            tu_slot[pos] = (int32_t)p;
            tu_ins[pos] = st == HT_INSERTED ? 1 : 0;
        }
    }
}

__global__ void k_lookup_spill_clear(const int32_t* __restrict__ flags, int64_t* __restrict__ spill_keys,
                                     uint8_t* __restrict__ spill_map, uint64_t cap) {
    if (flags[0] == 0) return;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < (int64_t)cap; i += stride) {
        spill_keys[i] = kEmpty;
        spill_map[i] = 0;
    }
}

// FULL survivors (no table slot) get a pseudo-slot in the spill set, a plain
// open-addressing set with an odd probe step (Theorem 1) and capacity 2n.
__global__ __launch_bounds__(kBlock) void k_lookup_spill_insert(
    const int32_t* __restrict__ flags, const int64_t* __restrict__ tu_keys, const int32_t* __restrict__ tu_count,
    int64_t ntiles, int64_t spill_base, int64_t* __restrict__ spill_keys, uint8_t* __restrict__ spill_map,
    uint64_t cap, int32_t* __restrict__ tu_slot) {
    if (flags[0] == 0) return;
    const uint64_t mask = cap - 1;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int cnt = tu_count[tile];
        for (int j = threadIdx.x; j < cnt; j += kBlock) {
            if (tu_slot[tile * kTile + j] >= 0) continue;
            const int64_t k = tu_keys[tile * kTile + j];
            const uint64_t h = mix64((uint64_t)k ^ 0x3C6EF372FE94F82Bull);
            uint64_t q = h & mask;
            const uint64_t stp = ((h >> 32) | 1ull) & mask;
            for (uint64_t probe = 0; probe <= mask; ++probe) {
                const int64_t cur = peek_key(&spill_keys[q]);
                if (cur == k) break;
                if (cur == kEmpty) {
                    const int64_t old = cas_key(&spill_keys[q], kEmpty, k);
                    if (old == kEmpty || old == k) break;
                }
                q = (q + stp) & mask;
            }
            if (spill_map[q] == 0) spill_map[q] = 1;
            tu_slot[tile * kTile + j] = (int32_t)(spill_base + (int64_t)q);
        }
    }
}

// Bytes of the touch maps -> one 64-bit word per 64 pseudo-slots.
__global__ void k_lookup_words(const uint8_t* __restrict__ mark, const uint8_t* __restrict__ spill_map,
                               const int32_t* __restrict__ flags, int64_t words_table, int64_t nwords,
                               uint64_t* __restrict__ word_bits, int32_t* __restrict__ word_cnt) {
    const bool spill = flags[0] != 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < nwords; w += stride) {
        uint64_t bits = 0;
        const uint8_t* src = nullptr;
        if (w < words_table) src = mark + w * 64;
        else if (spill) src = spill_map + (w - words_table) * 64;
        if (src) {
            const u32x4* v = reinterpret_cast<const u32x4*>(src);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 x = v[q];
                const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t m = xs[c] & 0x01010101u;        // bytes are 0 or 1
                    const uint32_t nib = (m | (m >> 7) | (m >> 14) | (m >> 21)) & 0xFu;
                    bits |= (uint64_t)nib << (16 * q + 4 * c);
                }
            }
        }
        word_bits[w] = bits;
        word_cnt[w] = __popcll(bits);
    }
}

// unique / slots / status for every marked pseudo-slot, in rank order; the
// table's map bytes of each non-empty word are zeroed again.
__global__ void k_lookup_emit(TableDev T, const int64_t* __restrict__ spill_keys, int64_t words_table,
                              int64_t nwords, const uint64_t* __restrict__ word_bits,
                              const int32_t* __restrict__ word_off, int64_t* __restrict__ unique,
                              int32_t* __restrict__ slots, uint8_t* __restrict__ status,
                              int64_t* __restrict__ n_unique) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_unique = word_off[nwords];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < nwords; w += stride) {
        uint64_t bits = word_bits[w];
        if (!bits) continue;
        int32_t r = word_off[w];
        const bool table_word = w < words_table;
        while (bits) {
            const int b = __builtin_ctzll(bits);
            bits &= bits - 1;
            const int64_t p = w * 64 + b;
            int64_t key;
            int32_t slot = -1;
            uint8_t st;
            if (table_word) {
                if (p < T.capacity) {
                    key = T.keys[p];
                    slot = (int32_t)p;
                    st = HT_FOUND;             // keys this call inserted are re-marked by the gather
                } else {
                    key = (p == T.capacity) ? kEmpty : kTomb;
                    st = HT_RESERVED;
                }
            } else {
                key = spill_keys[p - words_table * 64];
                st = HT_FULL;
            }
            unique[r] = key;
            slots[r] = slot;
            status[r] = st;
            ++r;
        }
        if (table_word) {
            u32x4 z;
            z.x = z.y = z.z = z.w = 0u;
            u32x4* m = reinterpret_cast<u32x4*>(T.mark + w * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) m[q] = z;
        }
    }
}

// Per survivor position: its dense id (rank of its pseudo-slot) into tu_gid,
// its table slot (or -1) back into tu_slot, and INSERTED status for keys it
// inserted.
__global__ void k_lookup_ids(int64_t M, const int32_t* __restrict__ tu_count, int64_t npos,
                             int32_t* __restrict__ tu_slot, const uint8_t* __restrict__ tu_ins,
                             const uint64_t* __restrict__ word_bits, const int32_t* __restrict__ word_off,
                             int32_t* __restrict__ tu_gid, uint8_t* __restrict__ status) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t pos = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; pos < npos; pos += stride) {
        if ((int)(pos & (kTile - 1)) >= tu_count[pos >> kTileLog2]) continue;
        const int64_t p = tu_slot[pos];
        const int64_t w = p >> 6;
        const int32_t gid = word_off[w] + __popcll(word_bits[w] & ((1ull << (p & 63)) - 1ull));
        tu_gid[pos] = gid;
        tu_slot[pos] = p < M ? (int32_t)p : -1;
        if (tu_ins[pos]) status[gid] = HT_INSERTED;
    }
}

// Per ID: its survivor record is tile-local (tile * kTile + local index), so
// the slot and id reads stay in a few cache lines per tile; then inverse and
// the row copy (TEAM lanes x 16 bytes per row, kUnroll rows in flight per
// team, non-temporal stores).
template <int TEAM>
__global__ __launch_bounds__(kBlock) void k_lookup_gather(TableDev T, const uint16_t* __restrict__ local, int64_t n,
                                                         const int32_t* __restrict__ tu_slot,
                                                         const int32_t* __restrict__ tu_gid,
                                                         int32_t* __restrict__ inverse, void* __restrict__ out) {
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    const int tl = threadIdx.x & (TEAM - 1);
    const int64_t team = (blockIdx.x * (int64_t)kBlock + threadIdx.x) / TEAM;
    const int64_t nteams = (int64_t)gridDim.x * kBlock / TEAM;
    if ((row_bytes & 15) == 0) {
        const int vpr = (int)(row_bytes >> 4);
        const u32x4* src = reinterpret_cast<const u32x4*>(T.rows);
        u32x4* dst = reinterpret_cast<u32x4*>(out);
        for (int64_t rb = team; rb < n; rb += nteams * kUnroll) {
            int32_t s[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t r = rb + u * nteams;
                s[u] = -1;
                if (r < n) {
                    const int64_t pos = ((r >> kTileLog2) << kTileLog2) + local[r];
                    s[u] = tu_slot[pos];
                    if (tl == 0) inverse[r] = tu_gid[pos];
                }
            }
            for (int v = tl; v < vpr; v += TEAM) {
                u32x4 val[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) val[u] = s[u] >= 0 ? src[(int64_t)s[u] * vpr + v] : zero4();
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int64_t r = rb + u * nteams;
                    if (r < n) __builtin_nontemporal_store(val[u], dst + r * vpr + v);
                }
            }
        }
    } else {
        // rows whose byte length is not a multiple of 16: one thread per element
        const int64_t stride = (int64_t)gridDim.x * kBlock;
        for (int64_t e = blockIdx.x * (int64_t)kBlock + threadIdx.x; e < n * T.dim; e += stride) {
            const int64_t r = e / T.dim;
            const int c = (int)(e - r * T.dim);
            const int64_t pos = ((r >> kTileLog2) << kTileLog2) + local[r];
            const int32_t s = tu_slot[pos];
            if (c == 0) inverse[r] = tu_gid[pos];
            if (T.elem_bytes == 4)
                ((uint32_t*)out)[e] = s >= 0 ? ((const uint32_t*)T.rows)[(int64_t)s * T.dim + c] : 0u;
            else
                ((uint16_t*)out)[e] = s >= 0 ? ((const uint16_t*)T.rows)[(int64_t)s * T.dim + c] : (uint16_t)0;
        }
    }
}

int team_for(int vpr) {
    int t = 1;
    while (t < vpr && t < 64) t <<= 1;
    return t;
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

size_t lookup_workspace_bytes(const htl_table* t, int64_t n) {
    if (!t) return 0;
    if (n < 0) n = 0;
    return lookup_layout(t->dev.capacity, n, nullptr).bytes;
}

htl_status ht_lookup_prepare(htl_table* t, const int64_t* keys, int64_t n, uint32_t step, int64_t* unique,
                             int64_t* n_unique_dev, int32_t* slots, uint8_t* status, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_lookup_prepare: null table");
    HTL_REQUIRE(t->capacity_log2 <= 30, "ht_lookup_prepare: needs capacity_log2 <= 30");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 28), "ht_lookup_prepare: n must be in [0, 2^28)");
    HTL_REQUIRE(n_unique_dev && aligned(n_unique_dev, 8), "ht_lookup_prepare: null or misaligned n_unique_dev");
    if (n == 0) {
        hipLaunchKernelGGL(k_write_zero_i64, dim3(1), dim3(1), 0, stream, n_unique_dev);
        return check_launch("ht_lookup_prepare");
    }
    HTL_REQUIRE(keys && unique && slots && status && ws, "ht_lookup_prepare: null pointer");
    HTL_REQUIRE(aligned(keys, 8) && aligned(unique, 8) && aligned(slots, 4) && aligned(ws, 256),
                "ht_lookup_prepare: misaligned pointer (ws needs 256 bytes)");
    const TableDev& T = t->dev;
    LookupWs w = lookup_layout(T.capacity, n, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "ht_lookup_prepare: workspace too small");
    const int64_t ntiles = ceil_div(n, kTile);
    const int64_t npos = ntiles * kTile;
    const unsigned gt = grid_for(ntiles, 1, 1 << 16);

    hipLaunchKernelGGL(k_lookup_reset, dim3(1), dim3(1), 0, stream, w.flags);
    hipLaunchKernelGGL(k_dedup_tile, dim3(gt), dim3(kTileThreads), 0, stream, keys, n, w.tu_keys, w.tu_count,
                       w.local);
    switch (probe_lanes()) {
#define HTL_CLAIM(GG)                                                                                        \
    hipLaunchKernelGGL(k_lookup_claim<GG>, dim3(grid_for(npos, kBlock / GG)), dim3(kBlock), 0, stream, T, w.tu_keys, \
                       w.tu_count, npos, step, w.tu_slot, w.tu_ins, w.flags)
        case 1: HTL_CLAIM(1); break;
        case 2: HTL_CLAIM(2); break;
        case 8: HTL_CLAIM(8); break;
        case 16: HTL_CLAIM(16); break;
        default: HTL_CLAIM(4); break;
#undef HTL_CLAIM
    }
    hipLaunchKernelGGL(k_lookup_spill_clear, dim3(grid_for((int64_t)w.spill_cap, 256 * 8, 1 << 14)), dim3(256), 0,
                       stream, w.flags, w.spill_keys, w.spill_map, w.spill_cap);
    hipLaunchKernelGGL(k_lookup_spill_insert, dim3(gt), dim3(kBlock), 0, stream, w.flags, w.tu_keys, w.tu_count,
                       ntiles, w.words_table * 64, w.spill_keys, w.spill_map, w.spill_cap, w.tu_slot);
    hipLaunchKernelGGL(k_lookup_words, dim3(grid_for(w.nwords, 256, 1 << 16)), dim3(256), 0, stream, T.mark,
                       w.spill_map, w.flags, w.words_table, w.nwords, w.word_bits, w.word_cnt);
    htl_status st = scan_exclusive_i32(w.word_cnt, w.word_off, w.nwords, nullptr, kScanIdentity, 1, w.scan_tmp,
                                       stream);
    if (st != HTL_OK) return st;
    hipLaunchKernelGGL(k_lookup_emit, dim3(grid_for(w.nwords, 256, 1 << 16)), dim3(256), 0, stream, T, w.spill_keys,
                       w.words_table, w.nwords, w.word_bits, w.word_off, unique, slots, status, n_unique_dev);
    return check_launch("ht_lookup_prepare");
}

htl_status ht_lookup_gather(htl_table* t, int64_t n, int32_t* inverse, uint8_t* status, void* out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "ht_lookup_gather: null table");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 28), "ht_lookup_gather: n must be in [0, 2^28)");
    if (n == 0) return HTL_OK;
    HTL_REQUIRE(inverse && status && out && ws, "ht_lookup_gather: null pointer");
    HTL_REQUIRE(aligned(inverse, 4) && aligned(out, 16) && aligned(ws, 256),
                "ht_lookup_gather: misaligned pointer (out needs 16 bytes, ws 256)");
    const TableDev& T = t->dev;
    LookupWs w = lookup_layout(T.capacity, n, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "ht_lookup_gather: workspace too small");
    const int64_t ntiles = ceil_div(n, kTile);
    const int64_t npos = ntiles * kTile;
    hipLaunchKernelGGL(k_lookup_ids, dim3(grid_for(npos, 256 * 4)), dim3(256), 0, stream, T.capacity, w.tu_count,
                       npos, w.tu_slot, w.tu_ins, w.word_bits, w.word_off, w.tu_gid, status);
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    const int vpr = (int)(row_bytes / 16);
    const int team = (row_bytes % 16) ? 1 : team_for(vpr);
    const unsigned grid = (row_bytes % 16) ? grid_for(n * T.dim, 256 * 4) : grid_for(n, (kBlock / team) * kUnroll);
    switch (team) {
#define HTL_GATHER(TT)                                                                                        \
    hipLaunchKernelGGL(k_lookup_gather<TT>, dim3(grid), dim3(kBlock), 0, stream, T, w.local, n, w.tu_slot, w.tu_gid, \
                       inverse, out)
        case 1: HTL_GATHER(1); break;
        case 2: HTL_GATHER(2); break;
        case 4: HTL_GATHER(4); break;
        case 8: HTL_GATHER(8); break;
        case 16: HTL_GATHER(16); break;
        case 32: HTL_GATHER(32); break;
        default: HTL_GATHER(64); break;
#undef HTL_GATHER
    }
    return check_launch("ht_lookup_gather");
}

htl_status ht_lookup(htl_table* t, const int64_t* keys, int64_t n, uint32_t step, int64_t* unique,
                     int32_t* inverse, int64_t* n_unique_dev, int32_t* slots, uint8_t* status, void* out,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
    htl_status st = ht_lookup_prepare(t, keys, n, step, unique, n_unique_dev, slots, status, ws, ws_bytes, stream);
    if (st != HTL_OK || n == 0) return st;
    HTL_REQUIRE(inverse && out, "ht_lookup: null inverse/out");
    return ht_lookup_gather(t, n, inverse, status, out, ws, ws_bytes, stream);
}

}  // extern "C"
