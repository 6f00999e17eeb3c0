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
// latency; the grid shrinks as kUnroll grows.  Event-timed on MI355X, IDs
// indexing slots directly, 2^22 IDs over a 2^24-slot table: 2 rows in flight
// 0.288 ms (256-byte rows) and 0.161 ms (128-byte rows), against 0.304 and
// 0.167 ms with 4 and 0.356 and 0.176 ms with 1.  Output rows are written
// with non-temporal stores: they are
// consumed by the next stage, not re-read here.  The pooled form is in
// pool.hip.
#include "pool.h"

namespace htl {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 2;

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
        // The index loads take no branch per row (a load under its own
        // guard waits for the one before it): past the end the last ID's
        // indices are loaded again and the row is dropped.  Same box, same
        // run: the large-table gather 0.373 -> 0.369 ms, the online (bf16)
        // gather 0.203 -> 0.192 ms.
        int32_t s[kUnroll];
        if (inverse) {
            int32_t iv[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t r = rb + u * nteams;
                iv[u] = inverse[r < n ? r : n - 1];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) s[u] = slots[iv[u]];
        } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t r = rb + u * nteams;
                s[u] = slots[r < n ? r : n - 1];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (rb + u * nteams >= n || s[u] >= M) s[u] = -1;   // past the end, or not a slot: zero row
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
    return launch_pooling(t->dev, t->dtype, vec, vpr, slots, inverse, n, offsets, nbags, out_dtype == HTL_BF16, out,
                          stream);
}

}  // extern "C"
