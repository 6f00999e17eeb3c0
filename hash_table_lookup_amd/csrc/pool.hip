// Embedding row gather with sum-pooling over multi-hot bags (the pooled form
// of emb_gather_pool; see gather.hip for the per-ID form).
//
// MTGenRec (arXiv 2505.12663), TL;DR: the lookup the dedup and the dynamic
// table serve.  With CSR bag offsets, each bag's rows are summed in fp32; the
// pooled row is written as fp32 or rounded to bf16 (nearest even).  Pooling is
// this library's reading for bag-shaped features: the pages do not describe
// it.  Rows are dtype[M][dim], read 16 bytes per lane.
#include "pool.h"

namespace htl {
namespace {

constexpr int kBlock = 256;
constexpr int kPoolUnroll = 8;             // IDs per team in flight (merged-tables step: 4 -> 1.40 ms, 8 -> 1.29, 16 -> 1.89)
constexpr int64_t kPoolBlocks = 1 << 14;   // workgroups of the wave-per-bag kernel (persistent grid)
// Workgroups of the team-per-bag kernel (persistent grid).  On the 26-table
// bf16 workload (1.70M bags): 2^13 / 2^14 / 2^15 / 2^16 / one team per bag
// 1.068 / 1.063 / 1.056 / 1.061 / 1.078 ms.
constexpr int64_t kPoolTeamBlocks = 1 << 15;

__device__ __forceinline__ u32x4 zero4() {
    u32x4 z;
    z.x = z.y = z.z = z.w = 0u;
    return z;
}

// A CSR position clamped to [0, n].
__device__ __forceinline__ int64_t clamp_pos(int32_t p, int64_t n) {
    return p < 0 ? 0 : (p > n ? n : (int64_t)p);
}

int team_for(int vpr) {
    int t = 1;
    while (t < vpr && t < 64) t <<= 1;
    return t;
}

// ------------------------------------------------------------- pooling --
// One wavefront per bag (rows of more than 32 vectors; shorter rows take
// k_pool_team below).  The wave splits into 64/TEAM teams; team q takes
// IDs q, q + 64/TEAM, ... of the bag, kPoolUnroll of them per round so that
// their three dependent loads (inverse, slot, row) overlap; every lane
// accumulates its 16-byte vectors in fp32; a butterfly over the teams then
// combines the partial sums.
template <int TEAM, int QMAX, bool IN_BF16>
__global__ __launch_bounds__(kBlock) void k_pool(const u32x4* __restrict__ rows, int vpr, int64_t M,
                                                const int32_t* __restrict__ slots,
                                                const int32_t* __restrict__ inverse, int64_t n,
                                                const int32_t* __restrict__ offsets, int64_t nbags,
                                                bool out_bf16, void* __restrict__ out) {
    constexpr int E = IN_BF16 ? 8 : 4;            // elements per 16-byte vector
    constexpr int TEAMS = 64 / TEAM;
    const int lane = lane_id();
    const int tl = lane & (TEAM - 1);
    const int q = lane / TEAM;
    const int64_t wave = (blockIdx.x * (int64_t)kBlock + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kBlock) >> 6;
    for (int64_t bag = wave; bag < nbags; bag += nwaves) {
        float acc[QMAX][E];
#pragma unroll
        for (int a = 0; a < QMAX; ++a)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[a][e] = 0.0f;
        // 64-bit positions: end may lie within TEAMS * kPoolUnroll of 2^31.
        // A bag is clamped to [0, n): offsets that break the CSR rules read
        // no ID outside the batch.
        const int64_t beg = clamp_pos(offsets[bag], n), end = clamp_pos(offsets[bag + 1], n);
        for (int64_t i0 = beg + q; i0 < end; i0 += TEAMS * kPoolUnroll) {
            // kPoolUnroll IDs per team in flight: inverse, then slots, then rows
            int32_t s[kPoolUnroll];
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u) {
                const int64_t i = i0 + u * TEAMS;
                s[u] = i < end ? (inverse ? inverse[i] : i) : -1;
            }
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u) {
                if (s[u] >= 0) s[u] = slots[s[u]];
                if (s[u] >= M) s[u] = -1;            // not a slot of this table: adds nothing
            }
#pragma unroll
            for (int a = 0; a < QMAX; ++a) {
                const int v = tl + a * TEAM;
                if (v >= vpr) break;
                u32x4 x[kPoolUnroll];
#pragma unroll
                for (int u = 0; u < kPoolUnroll; ++u) x[u] = s[u] >= 0 ? rows[(int64_t)s[u] * vpr + v] : zero4();
#pragma unroll
                for (int u = 0; u < kPoolUnroll; ++u) {
                    if (IN_BF16) {
                        const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            acc[a][2 * c] += bf16_lo(w[c]);
                            acc[a][2 * c + 1] += bf16_hi(w[c]);
                        }
                    } else {
                        acc[a][0] += __uint_as_float(x[u].x);
                        acc[a][1] += __uint_as_float(x[u].y);
                        acc[a][2] += __uint_as_float(x[u].z);
                        acc[a][3] += __uint_as_float(x[u].w);
                    }
                }
            }
        }
#pragma unroll
        for (int off = TEAM; off < 64; off <<= 1)
#pragma unroll
            for (int a = 0; a < QMAX; ++a)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[a][e] += __shfl_xor(acc[a][e], off);
        if (q != 0) continue;
#pragma unroll
        for (int a = 0; a < QMAX; ++a) {
            const int v = tl + a * TEAM;
            if (v >= vpr) break;
            const int64_t e0 = (bag * vpr + v) * E;     // first output element of this vector
            if (out_bf16) {
                uint32_t p[E / 2];
#pragma unroll
                for (int c = 0; c < E / 2; ++c)
                    p[c] = f32_to_bf16_bits(acc[a][2 * c]) | (f32_to_bf16_bits(acc[a][2 * c + 1]) << 16);
                uint16_t* o = (uint16_t*)out + e0;
                if (E == 8) {
                    u32x4 w;
                    w.x = p[0]; w.y = p[1]; w.z = p[2]; w.w = p[3];
                    __builtin_nontemporal_store(w, (u32x4*)o);
                } else {
                    __builtin_nontemporal_store(p[0], (uint32_t*)o);
                    __builtin_nontemporal_store(p[1], (uint32_t*)o + 1);
                }
            } else {
                float* o = (float*)out + e0;
#pragma unroll
                for (int c = 0; c < E / 4; ++c) {
                    u32x4 w;
                    w.x = __float_as_uint(acc[a][4 * c]);
                    w.y = __float_as_uint(acc[a][4 * c + 1]);
                    w.z = __float_as_uint(acc[a][4 * c + 2]);
                    w.w = __float_as_uint(acc[a][4 * c + 3]);
                    __builtin_nontemporal_store(w, (u32x4*)o + c);
                }
            }
        }
    }
}

// Element-wise pooling fallback: one thread per (bag, element), fp32 sums.
template <typename TIn>
__global__ void k_pool_elem(const TIn* __restrict__ rows, int dim, int64_t M, const int32_t* __restrict__ slots,
                            const int32_t* __restrict__ inverse, int64_t n, const int32_t* __restrict__ offsets,
                            int64_t nbags, bool in_bf16, bool out_bf16, void* __restrict__ out) {
    const int64_t total = nbags * dim;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t bag = e / dim;
        const int j = (int)(e - bag * dim);
        float acc = 0.0f;
        const int64_t end = clamp_pos(offsets[bag + 1], n);
        for (int64_t i = clamp_pos(offsets[bag], n); i < end; ++i) {
            const int32_t s = slots[inverse ? inverse[i] : i];
            if (s < 0 || s >= M) continue;
            const TIn x = rows[(int64_t)s * dim + j];
            acc += in_bf16 ? __uint_as_float((uint32_t)x << 16) : __uint_as_float((uint32_t)x);
        }
        if (out_bf16) ((uint16_t*)out)[e] = (uint16_t)f32_to_bf16_bits(acc);
        else ((float*)out)[e] = acc;
    }
}

// One team of TEAM lanes per bag, for rows of at most 32 vectors: the team
// walks its own bag kPoolUnroll IDs at a time and keeps the sum, so a
// wave keeps the rows of 64/TEAM bags in flight (a ~20-ID bag alone would
// leave a third of a wave's 32 row loads idle) and needs no combine across
// teams.  The pooling is bound by how many row loads are in flight: on the
// 26-table bf16 workload, 1.160 ms per launch with a wave per bag, 1.065 ms
// with a team per bag, 1.084 / 1.22 ms with 6 / 12 rows per team (12 costs
// two waves per SIMD), and a wave per bag at half the waves took 1.79 ms.
template <int TEAM, bool IN_BF16>
__global__ __launch_bounds__(kBlock) void k_pool_team(const u32x4* __restrict__ rows, int vpr, int64_t M,
                                                     const int32_t* __restrict__ slots,
                                                     const int32_t* __restrict__ inverse, int64_t n,
                                                     const int32_t* __restrict__ offsets, int64_t nbags,
                                                     bool out_bf16, void* __restrict__ out) {
    constexpr int E = IN_BF16 ? 8 : 4;
    const int tl = threadIdx.x & (TEAM - 1);
    const int64_t team = (blockIdx.x * (int64_t)kBlock + threadIdx.x) / TEAM;
    const int64_t nteams = (int64_t)gridDim.x * kBlock / TEAM;
    const bool lane_on = tl < vpr;
    for (int64_t bag = team; bag < nbags; bag += nteams) {
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.0f;
        const int64_t beg = clamp_pos(offsets[bag], n), end = clamp_pos(offsets[bag + 1], n);
        for (int64_t i0 = beg; i0 < end; i0 += kPoolUnroll) {
            int32_t sl[kPoolUnroll];
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u) {
                const int64_t i = i0 + u;
                sl[u] = i < end ? (inverse ? inverse[i] : (int32_t)i) : -1;
            }
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u) {
                if (sl[u] >= 0) sl[u] = slots[sl[u]];
                if (sl[u] >= M) sl[u] = -1;
            }
            u32x4 x[kPoolUnroll];
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u)
                x[u] = (lane_on && sl[u] >= 0) ? rows[(int64_t)sl[u] * vpr + tl] : zero4();
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u) {
                if (IN_BF16) {
                    const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        acc[2 * c] += bf16_lo(w[c]);
                        acc[2 * c + 1] += bf16_hi(w[c]);
                    }
                } else {
                    acc[0] += __uint_as_float(x[u].x);
                    acc[1] += __uint_as_float(x[u].y);
                    acc[2] += __uint_as_float(x[u].z);
                    acc[3] += __uint_as_float(x[u].w);
                }
            }
        }
        if (!lane_on) continue;
        const int64_t e0 = (bag * vpr + tl) * E;
        if (out_bf16) {
            uint32_t p[E / 2];
#pragma unroll
            for (int c = 0; c < E / 2; ++c) p[c] = f32_to_bf16_bits(acc[2 * c]) | (f32_to_bf16_bits(acc[2 * c + 1]) << 16);
            uint16_t* o = (uint16_t*)out + e0;
            if (E == 8) {
                u32x4 w;
                w.x = p[0]; w.y = p[1]; w.z = p[2]; w.w = p[3];
                __builtin_nontemporal_store(w, (u32x4*)o);
            } else {
                __builtin_nontemporal_store(p[0], (uint32_t*)o);
                __builtin_nontemporal_store(p[1], (uint32_t*)o + 1);
            }
        } else {
            float* o = (float*)out + e0;
#pragma unroll
            for (int c = 0; c < E / 4; ++c) {
                u32x4 w;
                w.x = __float_as_uint(acc[4 * c]);
                w.y = __float_as_uint(acc[4 * c + 1]);
                w.z = __float_as_uint(acc[4 * c + 2]);
                w.w = __float_as_uint(acc[4 * c + 3]);
                __builtin_nontemporal_store(w, (u32x4*)o + c);
            }
        }
    }
}

template <int TEAM, int QMAX>
void launch_pool(const TableDev& T, int vpr, const int32_t* slots, const int32_t* inverse, int64_t n,
                 const int32_t* offsets, int64_t nbags, bool out_bf16, void* out, hipStream_t s) {
    // A persistent grid (each team or wavefront strides over bags): on the
    // 1.7M-bag pooled workload, 16K workgroups ran 10% faster than one
    // wavefront per bag (426K workgroups); for the per-ID gather the full
    // grid was best.
    if (QMAX == 1 && TEAM <= 32) {
        const unsigned tgrid = grid_for(nbags, kBlock / TEAM, kPoolTeamBlocks);
        if (T.dtype == HTL_BF16)
            hipLaunchKernelGGL((k_pool_team<TEAM, true>), dim3(tgrid), dim3(kBlock), 0, s, (const u32x4*)T.rows,
                               vpr, T.capacity, slots, inverse, n, offsets, nbags, out_bf16, out);
        else
            hipLaunchKernelGGL((k_pool_team<TEAM, false>), dim3(tgrid), dim3(kBlock), 0, s, (const u32x4*)T.rows,
                               vpr, T.capacity, slots, inverse, n, offsets, nbags, out_bf16, out);
        return;
    }
    const unsigned grid = grid_for(nbags, kBlock / 64, kPoolBlocks);
    if (T.dtype == HTL_BF16)
        hipLaunchKernelGGL((k_pool<TEAM, QMAX, true>), dim3(grid), dim3(kBlock), 0, s, (const u32x4*)T.rows,
                           vpr, T.capacity, slots, inverse, n, offsets, nbags, out_bf16, out);
    else
        hipLaunchKernelGGL((k_pool<TEAM, QMAX, false>), dim3(grid), dim3(kBlock), 0, s, (const u32x4*)T.rows,
                           vpr, T.capacity, slots, inverse, n, offsets, nbags, out_bf16, out);
}

}  // namespace

htl_status launch_pooling(const TableDev& T, int dtype, bool vec, int vpr, const int32_t* slots,
                          const int32_t* inverse, int64_t n, const int32_t* offsets, int64_t nbags, bool out_bf16,
                          void* out, hipStream_t stream) {
    if (vec && vpr <= 256) {
        // One 16-byte vector per lane.  (With a wave per bag, narrower
        // teams with two vectors per lane, which keep a whole 20-ID bag in
        // flight in one round, measured 3% slower on the 26-table bf16
        // workload; a team per bag keeps more rows in flight instead.)
        switch (team_for(vpr)) {
            case 1: launch_pool<1, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream); break;
            case 2: launch_pool<2, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream); break;
            case 4: launch_pool<4, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream); break;
            case 8: launch_pool<8, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream); break;
            case 16: launch_pool<16, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream); break;
            case 32: launch_pool<32, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream); break;
            default:
                if (vpr <= 64) launch_pool<64, 1>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream);
                else if (vpr <= 128) launch_pool<64, 2>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream);
                else launch_pool<64, 4>(T, vpr, slots, inverse, n, offsets, nbags, out_bf16, out, stream);
                break;
        }
    } else {
        const unsigned grid = grid_for(nbags * T.dim, 256 * 4);
        if (dtype == HTL_F32)
            hipLaunchKernelGGL((k_pool_elem<uint32_t>), dim3(grid), dim3(256), 0, stream, (const uint32_t*)T.rows,
                               T.dim, T.capacity, slots, inverse, n, offsets, nbags, false, out_bf16, out);
        else
            hipLaunchKernelGGL((k_pool_elem<uint16_t>), dim3(grid), dim3(256), 0, stream, (const uint16_t*)T.rows,
                               T.dim, T.capacity, slots, inverse, n, offsets, nbags, true, out_bf16, out);
    }
    return check_launch("emb_gather_pool (pool)");
}

}  // namespace htl
