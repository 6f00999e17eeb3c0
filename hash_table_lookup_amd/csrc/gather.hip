// Embedding row gather with optional sum-pooling over multi-hot bags.
//
// MTGenRec (arXiv 2505.12663), TL;DR: the lookup the dedup and the dynamic
// table serve.  Without pooling, out[i] = rows[slots[inverse[i]]] (a bit
// copy; sequence items are embedded one per token, as in MTGR's feature
// tokenisation, arXiv 2505.18654 section 4).  With CSR bag offsets, each bag's
// rows are summed in fp32; the pooled row is written as fp32 or rounded to
// bf16 (nearest even).  Pooling is this library's reading for bag-shaped
// features: the pages do not describe it.
//
// Layout: rows are dtype[M][dim] by slot, read 16 bytes per lane.  A team of
// TEAM lanes (a power of two, at least one lane per 16-byte vector when the
// row has at most 64 of them) moves one row; a wavefront moves 64/TEAM rows
// per instruction.  Each team keeps kUnroll rows in flight to cover HBM
// latency.  Output rows are written with non-temporal stores: they are
// consumed by the next stage, not re-read here.
#include "htl_common.h"

namespace htl {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;
constexpr int kPoolUnroll = 4;         // IDs per team in flight in the pooling loop

__device__ __forceinline__ u32x4 zero4() {
    u32x4 z;
    z.x = z.y = z.z = z.w = 0u;
    return z;
}

template <int TEAM>
__global__ __launch_bounds__(kBlock) void k_gather(const u32x4* __restrict__ rows, int vpr, int64_t M,
                                                  const int32_t* __restrict__ slots,
                                                  const int32_t* __restrict__ inverse, int64_t n,
                                                  u32x4* __restrict__ out) {
    const int tl = threadIdx.x & (TEAM - 1);
    const int64_t team = (blockIdx.x * (int64_t)kBlock + threadIdx.x) / TEAM;
    const int64_t nteams = (int64_t)gridDim.x * kBlock / TEAM;
    for (int64_t rb = team; rb < n; rb += nteams * kUnroll) {
        int32_t s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t r = rb + u * nteams;
            s[u] = -1;
            if (r < n) s[u] = slots[inverse ? inverse[r] : r];
            if (s[u] >= M) s[u] = -1;            // not a slot of this table: zero row
        }
        for (int v = tl; v < vpr; v += TEAM) {
            u32x4 val[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                val[u] = s[u] >= 0 ? rows[(int64_t)s[u] * vpr + v] : zero4();
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t r = rb + u * nteams;
                if (r < n) __builtin_nontemporal_store(val[u], out + r * vpr + v);
            }
        }
    }
}

// bf16 table -> fp32 output (exact widening), 8 elements per input vector.
template <int TEAM>
__global__ __launch_bounds__(kBlock) void k_gather_widen(const u32x4* __restrict__ rows, int vpr, int64_t M,
                                                        const int32_t* __restrict__ slots,
                                                        const int32_t* __restrict__ inverse, int64_t n,
                                                        u32x4* __restrict__ out) {
    const int tl = threadIdx.x & (TEAM - 1);
    const int64_t team = (blockIdx.x * (int64_t)kBlock + threadIdx.x) / TEAM;
    const int64_t nteams = (int64_t)gridDim.x * kBlock / TEAM;
    for (int64_t r = team; r < n; r += nteams) {
        int32_t s = slots[inverse ? inverse[r] : r];
        if (s >= M) s = -1;
        for (int v = tl; v < vpr; v += TEAM) {
            const u32x4 x = s >= 0 ? rows[(int64_t)s * vpr + v] : zero4();
            u32x4 a, b;
            a.x = x.x << 16; a.y = x.x & 0xFFFF0000u; a.z = x.y << 16; a.w = x.y & 0xFFFF0000u;
            b.x = x.z << 16; b.y = x.z & 0xFFFF0000u; b.z = x.w << 16; b.w = x.w & 0xFFFF0000u;
            __builtin_nontemporal_store(a, out + r * (2 * vpr) + 2 * v);
            __builtin_nontemporal_store(b, out + r * (2 * vpr) + 2 * v + 1);
        }
    }
}

// Element-wise fallback for rows whose byte length is not a multiple of 16.
template <typename TIn, typename TOut>
__global__ void k_gather_elem(const TIn* __restrict__ rows, int dim, int64_t M, const int32_t* __restrict__ slots,
                              const int32_t* __restrict__ inverse, int64_t n, TOut* __restrict__ out,
                              bool widen_bf16) {
    const int64_t total = n * dim;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t r = e / dim;
        const int j = (int)(e - r * dim);
        const int32_t s = slots[inverse ? inverse[r] : r];
        TIn x = (s >= 0 && s < M) ? rows[(int64_t)s * dim + j] : (TIn)0;
        if (widen_bf16) out[e] = (TOut)__float_as_uint(__uint_as_float((uint32_t)x << 16));
        else out[e] = (TOut)x;
    }
}

// ------------------------------------------------------------- pooling --
// One wavefront per bag.  The wave splits into 64/TEAM teams; team q takes
// IDs q, q + 64/TEAM, ... of the bag, kPoolUnroll of them per round so that
// their three dependent loads (inverse, slot, row) overlap; every lane
// accumulates its 16-byte vectors in fp32; a butterfly over the teams then
// combines the partial sums.
template <int TEAM, int QMAX, bool IN_BF16>
__global__ __launch_bounds__(kBlock) void k_pool(const u32x4* __restrict__ rows, int vpr, int64_t M,
                                                const int32_t* __restrict__ slots,
                                                const int32_t* __restrict__ inverse,
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
        const int32_t beg = offsets[bag], end = offsets[bag + 1];
        for (int32_t i0 = beg + q; i0 < end; i0 += TEAMS * kPoolUnroll) {
            // kPoolUnroll IDs per team in flight: inverse, then slots, then rows
            int32_t s[kPoolUnroll];
#pragma unroll
            for (int u = 0; u < kPoolUnroll; ++u) {
                const int32_t i = i0 + u * TEAMS;
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
                            const int32_t* __restrict__ inverse, const int32_t* __restrict__ offsets,
                            int64_t nbags, bool in_bf16, bool out_bf16, void* __restrict__ out) {
    const int64_t total = nbags * dim;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t bag = e / dim;
        const int j = (int)(e - bag * dim);
        float acc = 0.0f;
        for (int32_t i = offsets[bag]; i < offsets[bag + 1]; ++i) {
            const int32_t s = slots[inverse ? inverse[i] : i];
            if (s < 0 || s >= M) continue;
            const TIn x = rows[(int64_t)s * dim + j];
            acc += in_bf16 ? __uint_as_float((uint32_t)x << 16) : __uint_as_float((uint32_t)x);
        }
        if (out_bf16) ((uint16_t*)out)[e] = (uint16_t)f32_to_bf16_bits(acc);
        else ((float*)out)[e] = acc;
    }
}

int team_for(int vpr) {
    int t = 1;
    while (t < vpr && t < 64) t <<= 1;
    return t;
}

template <int TEAM>
void launch_gather(const TableDev& T, int vpr, const int32_t* slots, const int32_t* inverse, int64_t n,
                   void* out, bool widen, hipStream_t s) {
    const unsigned grid = grid_for(n, (kBlock / TEAM) * (widen ? 1 : kUnroll));
    if (widen)
        hipLaunchKernelGGL(k_gather_widen<TEAM>, dim3(grid), dim3(kBlock), 0, s, (const u32x4*)T.rows, vpr,
                           T.capacity, slots, inverse, n, (u32x4*)out);
    else
        hipLaunchKernelGGL(k_gather<TEAM>, dim3(grid), dim3(kBlock), 0, s, (const u32x4*)T.rows, vpr,
                           T.capacity, slots, inverse, n, (u32x4*)out);
}

template <int TEAM, int QMAX>
void launch_pool(const TableDev& T, int vpr, const int32_t* slots, const int32_t* inverse,
                 const int32_t* offsets, int64_t nbags, bool out_bf16, void* out, hipStream_t s) {
    const unsigned grid = grid_for(nbags, kBlock / 64);
    if (T.dtype == HTL_BF16)
        hipLaunchKernelGGL((k_pool<TEAM, QMAX, true>), dim3(grid), dim3(kBlock), 0, s, (const u32x4*)T.rows,
                           vpr, T.capacity, slots, inverse, offsets, nbags, out_bf16, out);
    else
        hipLaunchKernelGGL((k_pool<TEAM, QMAX, false>), dim3(grid), dim3(kBlock), 0, s, (const u32x4*)T.rows,
                           vpr, T.capacity, slots, inverse, offsets, nbags, out_bf16, out);
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

htl_status emb_gather_pool(const htl_table* t, const int32_t* slots, const int32_t* inverse, int64_t n,
                           const int32_t* offsets, int64_t nbags, htl_dtype out_dtype, void* out,
                           hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "emb_gather_pool: null table");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "emb_gather_pool: n must be in [0, 2^31)");
    HTL_REQUIRE(out_dtype == HTL_F32 || out_dtype == HTL_BF16, "emb_gather_pool: bad out_dtype");
    const TableDev& T = t->dev;
    const int64_t row_bytes = (int64_t)T.dim * T.elem_bytes;
    const bool vec = (row_bytes % 16) == 0;
    const int vpr = (int)(row_bytes / 16);
    if (offsets == nullptr) {
        HTL_REQUIRE(out_dtype == t->dtype || (t->dtype == HTL_BF16 && out_dtype == HTL_F32),
                    "emb_gather_pool: without pooling out_dtype must be the table dtype or fp32");
        if (n == 0) return HTL_OK;
        HTL_REQUIRE(slots && out, "emb_gather_pool: null slots/out");
        HTL_REQUIRE(aligned(slots, 4) && (!inverse || aligned(inverse, 4)) && aligned(out, 16),
                    "emb_gather_pool: misaligned pointer (out needs 16 bytes)");
        const bool widen = out_dtype != t->dtype;
        if (vec) {
            switch (team_for(vpr)) {
                case 1: launch_gather<1>(T, vpr, slots, inverse, n, out, widen, stream); break;
                case 2: launch_gather<2>(T, vpr, slots, inverse, n, out, widen, stream); break;
                case 4: launch_gather<4>(T, vpr, slots, inverse, n, out, widen, stream); break;
                case 8: launch_gather<8>(T, vpr, slots, inverse, n, out, widen, stream); break;
                case 16: launch_gather<16>(T, vpr, slots, inverse, n, out, widen, stream); break;
                case 32: launch_gather<32>(T, vpr, slots, inverse, n, out, widen, stream); break;
                default: launch_gather<64>(T, vpr, slots, inverse, n, out, widen, stream); break;
            }
        } else {
            const unsigned grid = grid_for(n * T.dim, 256 * 4);
            if (t->dtype == HTL_F32)
                hipLaunchKernelGGL((k_gather_elem<uint32_t, uint32_t>), dim3(grid), dim3(256), 0, stream,
                                   (const uint32_t*)T.rows, T.dim, T.capacity, slots, inverse, n, (uint32_t*)out, false);
            else if (!widen)
                hipLaunchKernelGGL((k_gather_elem<uint16_t, uint16_t>), dim3(grid), dim3(256), 0, stream,
                                   (const uint16_t*)T.rows, T.dim, T.capacity, slots, inverse, n, (uint16_t*)out, false);
            else
                hipLaunchKernelGGL((k_gather_elem<uint16_t, uint32_t>), dim3(grid), dim3(256), 0, stream,
                                   (const uint16_t*)T.rows, T.dim, T.capacity, slots, inverse, n, (uint32_t*)out, true);
        }
        return check_launch("emb_gather_pool (gather)");
    }
    HTL_REQUIRE(nbags >= 0 && nbags < ((int64_t)1 << 31), "emb_gather_pool: nbags out of range");
    if (nbags == 0) return HTL_OK;
    HTL_REQUIRE(out && (n == 0 || slots), "emb_gather_pool: null slots/out");
    HTL_REQUIRE(aligned(offsets, 4) && (!slots || aligned(slots, 4)) && (!inverse || aligned(inverse, 4)) &&
                    aligned(out, 16),
                "emb_gather_pool: misaligned pointer (out needs 16 bytes)");
    const bool out_bf16 = out_dtype == HTL_BF16;
    if (vec && vpr <= 256) {
        // One 16-byte vector per lane.  (Narrower teams with two vectors
        // per lane, which keep a whole 20-ID bag in flight in one round,
        // measured 3% slower on the 26-table bf16 workload: the pooled rows
        // come from cache and the loop is not latency-bound.)
        switch (team_for(vpr)) {
            case 1: launch_pool<1, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream); break;
            case 2: launch_pool<2, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream); break;
            case 4: launch_pool<4, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream); break;
            case 8: launch_pool<8, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream); break;
            case 16: launch_pool<16, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream); break;
            case 32: launch_pool<32, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream); break;
            default:
                if (vpr <= 64) launch_pool<64, 1>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream);
                else if (vpr <= 128) launch_pool<64, 2>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream);
                else launch_pool<64, 4>(T, vpr, slots, inverse, offsets, nbags, out_bf16, out, stream);
                break;
        }
    } else {
        const unsigned grid = grid_for(nbags * T.dim, 256 * 4);
        if (t->dtype == HTL_F32)
            hipLaunchKernelGGL((k_pool_elem<uint32_t>), dim3(grid), dim3(256), 0, stream, (const uint32_t*)T.rows,
                               T.dim, T.capacity, slots, inverse, offsets, nbags, false, out_bf16, out);
        else
            hipLaunchKernelGGL((k_pool_elem<uint16_t>), dim3(grid), dim3(256), 0, stream, (const uint16_t*)T.rows,
                               T.dim, T.capacity, slots, inverse, offsets, nbags, true, out_bf16, out);
    }
    return check_launch("emb_gather_pool (pool)");
}

}  // extern "C"
