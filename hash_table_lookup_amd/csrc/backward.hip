// Backward of the deduplicated lookup: gradient segment-sum per unique key,
// and the row-wise Adam update of the rows a batch hit.
//
// The pages describe the forward dedup (MTGenRec arXiv 2505.12663 TL;DR;
// MTGR arXiv 2505.18654 section 5, "Embedding Lookup"); its backward is the
// adjoint: the gradient of a unique row is the sum of the gradients of all IDs
// that mapped to it.  Adam (Kingma & Ba) with per-call bias corrections
// follows the TensorFlow article's section 3.2, where Adam's beta terms are
// kept local to each server instead of shared.
//
// Segment sum, without sorting the 4-byte-per-ID gradients' owners globally:
//   count  -- per tile of IDs, an LDS hash of the inverse values counts each
//             local unique; one global atomicAdd per (tile, unique) reserves
//             the tile's places inside that unique's segment (hot keys cost
//             one atomic per tile, not one per ID);
//   scan   -- segment offsets = exclusive prefix sum of the counts;
//   fill   -- perm[offset[u] + place] = i (CSR of IDs grouped by unique);
//   small  -- one wavefront per segment of <= kSmallMax IDs sums its rows;
//   large  -- longer segments (Zipf's head: the hottest key of a 2^23-ID
//             Zipf(1.2) batch owns ~18% of all rows) are cut into kChunk-row
//             chunks, one workgroup each, and the chunk partials are then
//             added in chunk order.
// Accumulation is fp32.  The order of IDs inside a segment depends on atomic
// order, so sums are reproducible only up to fp32 rounding.
#include <cmath>

#include "scan.h"

namespace htl {
namespace {

constexpr int kCTile = 2048;               // IDs per counting tile
constexpr int kCThreads = 256;
constexpr int kCPerThread = kCTile / kCThreads;
constexpr int kCCap = 2 * kCTile;          // LDS hash slots
constexpr int kCCapLog2 = 12;
constexpr int kSmallMax = 256;             // longest segment summed by one wavefront
constexpr int kChunk = 1024;               // rows per workgroup in long segments
constexpr int kRBlock = 256;

struct SegWs {
    int32_t* counts;       // [u_max]
    int32_t* seg_off;      // [u_max + 1]
    int32_t* rel;          // [n]
    int32_t* perm;         // [n]
    int32_t* large;        // [large_max]
    int32_t* large_off;    // [large_max + 1]
    unsigned long long* n_large;
    void* scan_tmp;
    float* partial;        // [max_chunks][dim]
    int64_t large_max, max_chunks;
    size_t bytes;
};

SegWs seg_layout(int64_t n, int64_t u_max, int dim, char* base) {
    SegWs w{};
    w.large_max = n / (kSmallMax + 1) + 1;
    w.max_chunks = n / kChunk + w.large_max;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    w.counts = (int32_t*)take((size_t)u_max * 4);
    w.seg_off = (int32_t*)take((size_t)(u_max + 1) * 4);
    w.rel = (int32_t*)take((size_t)n * 4);
    w.perm = (int32_t*)take((size_t)n * 4);
    w.large = (int32_t*)take((size_t)w.large_max * 4);
    w.large_off = (int32_t*)take((size_t)(w.large_max + 1) * 4);
    w.n_large = (unsigned long long*)take(8);
    w.scan_tmp = take(scan_temp_bytes(u_max));
    w.partial = (float*)take((size_t)w.max_chunks * dim * 4);
    w.bytes = off;
    return w;
}

__device__ __forceinline__ int64_t dev_count(int64_t n_max, const int64_t* n_dev) {
    if (!n_dev) return n_max;
    const int64_t c = *n_dev;
    return c < 0 ? 0 : (c < n_max ? c : n_max);
}

__global__ void k_seg_zero(int32_t* __restrict__ counts, int64_t u_max, const int64_t* __restrict__ n_dev,
                           unsigned long long* __restrict__ n_large) {
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < U; i += stride) counts[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_large = 0ull;
}

__global__ __launch_bounds__(kCThreads) void k_seg_count(const int32_t* __restrict__ inverse, int64_t n,
                                                        int64_t u_max, const int64_t* __restrict__ n_dev,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ rel) {
    __shared__ int32_t s_u[kCCap];
    __shared__ int32_t s_cnt[kCCap];
    __shared__ int32_t s_base[kCCap];
    const int tid = threadIdx.x;
    const int64_t U = dev_count(u_max, n_dev);
    for (int64_t tile = blockIdx.x; tile * kCTile < n; tile += gridDim.x) {
        const int64_t base = tile * kCTile;
        for (int i = tid; i < kCCap; i += kCThreads) {
            s_u[i] = -1;
            s_cnt[i] = 0;
        }
        __syncthreads();
        int pos[kCPerThread], rank[kCPerThread];
#pragma unroll
        for (int j = 0; j < kCPerThread; ++j) {
            const int64_t idx = base + j * kCThreads + tid;
            pos[j] = -1;
            rank[j] = 0;
            if (idx >= n) continue;
            const int32_t u = inverse[idx];
            if (u < 0 || u >= U) continue;       // outside [0, U): contributes nowhere
            const uint32_t h = (uint32_t)u * 0x9E3779B1u;
            uint32_t p = h >> (32 - kCCapLog2);
            const uint32_t stp = ((h >> 7) | 1u) & (kCCap - 1);
            for (int probe = 0; probe < kCCap; ++probe) {
                const int32_t old = atomicCAS(&s_u[p], -1, u);
                if (old == -1 || old == u) break;
                p = (p + stp) & (kCCap - 1);
            }
            pos[j] = (int)p;
            rank[j] = atomicAdd(&s_cnt[p], 1);
        }
        __syncthreads();
        for (int i = tid; i < kCCap; i += kCThreads) {
            const int32_t u = s_u[i];
            if (u >= 0) s_base[i] = atomicAdd(&counts[u], s_cnt[i]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kCPerThread; ++j) {
            const int64_t idx = base + j * kCThreads + tid;
            if (pos[j] >= 0) rel[idx] = s_base[pos[j]] + rank[j];
        }
        __syncthreads();
    }
}

__global__ void k_seg_fill(const int32_t* __restrict__ inverse, const int32_t* __restrict__ rel, int64_t n,
                           int64_t u_max, const int64_t* __restrict__ n_dev, const int32_t* __restrict__ seg_off,
                           int32_t* __restrict__ perm) {
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        const int32_t u = inverse[i];
        if (u >= 0 && u < U) perm[seg_off[u] + rel[i]] = (int32_t)i;
    }
}

// Sums rows perm[beg..end) of `grad` into acc, TEAM lanes per row, the
// TEAMS teams of `nthreads` lanes taking every TEAMS-th row.
template <int TEAM, int QMAX>
__device__ __forceinline__ void sum_rows(const u32x4* __restrict__ grad, int vpr, const int32_t* __restrict__ perm,
                                         int32_t beg, int32_t end, int team, int teams, int tl,
                                         float (&acc)[QMAX][4]) {
    constexpr int U = 4;
    for (int32_t i0 = beg + team; i0 < end; i0 += teams * U) {
        int32_t r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t i = i0 + u * teams;
            r[u] = i < end ? perm[i] : -1;
        }
#pragma unroll
        for (int a = 0; a < QMAX; ++a) {
            const int v = tl + a * TEAM;
            if (v >= vpr) break;
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (r[u] >= 0) x[u] = grad[(int64_t)r[u] * vpr + v];
                else x[u].x = x[u].y = x[u].z = x[u].w = 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc[a][0] += __uint_as_float(x[u].x);
                acc[a][1] += __uint_as_float(x[u].y);
                acc[a][2] += __uint_as_float(x[u].z);
                acc[a][3] += __uint_as_float(x[u].w);
            }
        }
    }
}

template <int TEAM, int QMAX>
__device__ __forceinline__ void store_row(float* __restrict__ dst, int vpr, int tl, const float (&acc)[QMAX][4]) {
#pragma unroll
    for (int a = 0; a < QMAX; ++a) {
        const int v = tl + a * TEAM;
        if (v >= vpr) break;
        u32x4 w;
        w.x = __float_as_uint(acc[a][0]);
        w.y = __float_as_uint(acc[a][1]);
        w.z = __float_as_uint(acc[a][2]);
        w.w = __float_as_uint(acc[a][3]);
        reinterpret_cast<u32x4*>(dst)[v] = w;
    }
}

// One wavefront per segment; segments longer than kSmallMax are listed for
// the chunked path instead.
template <int TEAM, int QMAX>
__global__ __launch_bounds__(kRBlock) void k_seg_small(const u32x4* __restrict__ grad, int vpr,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ seg_off, int64_t u_max,
                                                      const int64_t* __restrict__ n_dev, float* __restrict__ out,
                                                      int32_t* __restrict__ large,
                                                      unsigned long long* __restrict__ n_large) {
    const int64_t U = dev_count(u_max, n_dev);
    const int lane = lane_id();
    const int tl = lane & (TEAM - 1);
    const int team = lane / TEAM;
    constexpr int TEAMS = 64 / TEAM;
    const int64_t wave = (blockIdx.x * (int64_t)kRBlock + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kRBlock) >> 6;
    for (int64_t u = wave; u < U; u += nwaves) {
        const int32_t beg = seg_off[u], end = seg_off[u + 1];
        if (end - beg > kSmallMax) {
            if (lane == 0) large[atomicAdd(n_large, 1ull)] = (int32_t)u;
            continue;
        }
        float acc[QMAX][4];
#pragma unroll
        for (int a = 0; a < QMAX; ++a) acc[a][0] = acc[a][1] = acc[a][2] = acc[a][3] = 0.0f;
        sum_rows<TEAM, QMAX>(grad, vpr, perm, beg, end, team, TEAMS, tl, acc);
#pragma unroll
        for (int off = TEAM; off < 64; off <<= 1)
#pragma unroll
            for (int a = 0; a < QMAX; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[a][e] += __shfl_xor(acc[a][e], off);
        if (team == 0) store_row<TEAM, QMAX>(out + u * (int64_t)vpr * 4, vpr, tl, acc);
    }
}

// One block: large_off = exclusive scan of ceil(count / kChunk) over the list.
__global__ __launch_bounds__(1024) void k_large_scan(const int32_t* __restrict__ large,
                                                    const unsigned long long* __restrict__ n_large,
                                                    const int32_t* __restrict__ seg_off,
                                                    int32_t* __restrict__ large_off) {
    __shared__ int32_t s_warp[16];
    __shared__ int32_t s_carry;
    const int64_t nl = (int64_t)*n_large;
    if (threadIdx.x == 0) s_carry = 0;
    __syncthreads();
    for (int64_t b0 = 0; b0 <= nl; b0 += 1024) {
        const int64_t i = b0 + threadIdx.x;
        int32_t x = 0;
        if (i < nl) {
            const int32_t u = large[i];
            x = (seg_off[u + 1] - seg_off[u] + kChunk - 1) / kChunk;
        }
        const int lane = lane_id();
        const int wid = threadIdx.x >> 6;
        int32_t incl = x;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == 63) s_warp[wid] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wid) before += s_warp[w];
            total += s_warp[w];
        }
        const int32_t carry = s_carry;
        if (i <= nl) large_off[i] = carry + before + incl - x;
        __syncthreads();
        if (threadIdx.x == 0) s_carry = carry + total;
        __syncthreads();
    }
}

// One workgroup per chunk of a long segment -> partial[chunk].
template <int TEAM, int QMAX>
__global__ __launch_bounds__(kRBlock) void k_large_reduce(const u32x4* __restrict__ grad, int vpr,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ seg_off,
                                                         const int32_t* __restrict__ large,
                                                         const unsigned long long* __restrict__ n_large,
                                                         const int32_t* __restrict__ large_off, int64_t max_chunks,
                                                         float* __restrict__ partial) {
    constexpr int TEAMS = kRBlock / TEAM;
    __shared__ float s_acc[TEAMS][QMAX * TEAM * 4];
    const int64_t nl = (int64_t)*n_large;
    const int32_t total = large_off[nl];
    const int tl = threadIdx.x & (TEAM - 1);
    const int team = threadIdx.x / TEAM;
    for (int64_t c = blockIdx.x; c < total && c < max_chunks; c += gridDim.x) {
        // the list entry owning chunk c: last i with large_off[i] <= c
        int64_t lo = 0, hi = nl;              // large_off[lo] <= c < large_off[hi]
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (large_off[mid] <= c) lo = mid;
            else hi = mid;
        }
        const int32_t u = large[lo];
        const int32_t part = (int32_t)(c - large_off[lo]);
        const int32_t beg = seg_off[u] + part * kChunk;
        const int32_t end = min(seg_off[u + 1], beg + kChunk);
        float acc[QMAX][4];
#pragma unroll
        for (int a = 0; a < QMAX; ++a) acc[a][0] = acc[a][1] = acc[a][2] = acc[a][3] = 0.0f;
        sum_rows<TEAM, QMAX>(grad, vpr, perm, beg, end, team, TEAMS, tl, acc);
#pragma unroll
        for (int a = 0; a < QMAX; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) s_acc[team][(a * TEAM + tl) * 4 + e] = acc[a][e];
        __syncthreads();
        float* dst = partial + c * (int64_t)vpr * 4;
        for (int e = threadIdx.x; e < vpr * 4; e += kRBlock) {
            const int a = (e / 4) / TEAM, l = (e / 4) % TEAM;
            float s = 0.0f;
            for (int q = 0; q < TEAMS; ++q) s += s_acc[q][(a * TEAM + l) * 4 + (e & 3)];
            dst[e] = s;
        }
        __syncthreads();
    }
}

// One workgroup per long segment: out[u] = sum of its chunk partials in order.
__global__ __launch_bounds__(kRBlock) void k_large_combine(const float* __restrict__ partial, int dim,
                                                          const int32_t* __restrict__ large,
                                                          const unsigned long long* __restrict__ n_large,
                                                          const int32_t* __restrict__ large_off,
                                                          float* __restrict__ out) {
    const int64_t nl = (int64_t)*n_large;
    for (int64_t i = blockIdx.x; i < nl; i += gridDim.x) {
        const int32_t u = large[i];
        const int32_t c0 = large_off[i], c1 = large_off[i + 1];
        for (int e = threadIdx.x; e < dim; e += kRBlock) {
            float s = 0.0f;
            for (int32_t c = c0; c < c1; ++c) s += partial[(int64_t)c * dim + e];
            out[(int64_t)u * dim + e] = s;
        }
    }
}

// Element-wise fallback (dim not a multiple of 4): one thread per (u, j).
__global__ void k_seg_elem(const float* __restrict__ grad, int dim, const int32_t* __restrict__ perm,
                           const int32_t* __restrict__ seg_off, int64_t u_max, const int64_t* __restrict__ n_dev,
                           float* __restrict__ out) {
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < U * dim; e += stride) {
        const int64_t u = e / dim;
        const int j = (int)(e - u * dim);
        float s = 0.0f;
        for (int32_t i = seg_off[u]; i < seg_off[u + 1]; ++i) s += grad[(int64_t)perm[i] * dim + j];
        out[e] = s;
    }
}

template <int TEAM, int QMAX>
void launch_reduce(const float* grad, int vpr, const SegWs& w, int64_t u_max, const int64_t* n_dev, float* out,
                   hipStream_t s) {
    hipLaunchKernelGGL((k_seg_small<TEAM, QMAX>), dim3(grid_for(u_max, kRBlock / 64)), dim3(kRBlock), 0, s,
                       (const u32x4*)grad, vpr, w.perm, w.seg_off, u_max, n_dev, out, w.large, w.n_large);
    hipLaunchKernelGGL(k_large_scan, dim3(1), dim3(1024), 0, s, w.large, w.n_large, w.seg_off, w.large_off);
    hipLaunchKernelGGL((k_large_reduce<TEAM, QMAX>), dim3(grid_for(w.max_chunks, 1, 1 << 16)), dim3(kRBlock), 0,
                       s, (const u32x4*)grad, vpr, w.perm, w.seg_off, w.large, w.n_large, w.large_off,
                       w.max_chunks, w.partial);
    hipLaunchKernelGGL(k_large_combine, dim3(grid_for(w.large_max, 1, 1 << 14)), dim3(kRBlock), 0, s, w.partial,
                       vpr * 4, w.large, w.n_large, w.large_off, out);
}

// ---------------------------------------------------------------- Adam --
#pragma clang fp contract(off)
__global__ void k_adam(float* __restrict__ theta, float* __restrict__ m, float* __restrict__ v, int dim, int64_t M,
                       const int32_t* __restrict__ slots, const float* __restrict__ g, int64_t u_max,
                       const int64_t* __restrict__ n_dev, float lr, float b1, float b2, float eps, float c1,
                       float c2) {
    const int64_t U = dev_count(u_max, n_dev);
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < U * dim; e += stride) {
        const int64_t u = e / dim;
        const int j = (int)(e - u * dim);
        const int32_t s = slots[u];
        if (s < 0 || s >= M) continue;
        const int64_t o = (int64_t)s * dim + j;
        const float gj = g[e];
        const float mj = b1 * m[o] + omb1 * gj;
        const float vj = b2 * v[o] + omb2 * (gj * gj);
        const float mhat = mj / c1;
        const float vhat = vj / c2;
        theta[o] = theta[o] - lr * (mhat / (sqrtf(vhat) + eps));
        m[o] = mj;
        v[o] = vj;
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

size_t segsum_workspace_bytes(int64_t n, int64_t u_max, int dim) {
    if (n < 0) n = 0;
    if (u_max < 0) u_max = 0;
    if (dim < 1) dim = 1;
    return seg_layout(n, u_max, dim, nullptr).bytes;
}

htl_status emb_grad_segment_sum(const float* grad, const int32_t* inverse, int64_t n,
                                const int64_t* n_unique_dev, int64_t u_max, int dim, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "emb_grad_segment_sum: n must be in [0, 2^31)");
    HTL_REQUIRE(u_max >= 0 && u_max <= n, "emb_grad_segment_sum: u_max must be in [0, n]");
    HTL_REQUIRE(dim >= 1 && dim <= 65536, "emb_grad_segment_sum: dim must be in [1, 65536]");
    if (n == 0 || u_max == 0) return HTL_OK;
    HTL_REQUIRE(grad && inverse && out && ws, "emb_grad_segment_sum: null pointer");
    HTL_REQUIRE(aligned(grad, 16) && aligned(out, 16) && aligned(inverse, 4) && aligned(ws, 256) &&
                    (!n_unique_dev || aligned(n_unique_dev, 8)),
                "emb_grad_segment_sum: misaligned pointer (grad/out need 16 bytes, ws 256)");
    SegWs w = seg_layout(n, u_max, dim, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "emb_grad_segment_sum: workspace too small");

    hipLaunchKernelGGL(k_seg_zero, dim3(grid_for(u_max, 256 * 4, 1 << 14)), dim3(256), 0, stream, w.counts, u_max,
                       n_unique_dev, w.n_large);
    hipLaunchKernelGGL(k_seg_count, dim3(grid_for(ceil_div(n, kCTile), 1, 1 << 16)), dim3(kCThreads), 0, stream,
                       inverse, n, u_max, n_unique_dev, w.counts, w.rel);
    htl_status st = scan_exclusive_i32(w.counts, w.seg_off, u_max, n_unique_dev, kScanIdentity, 1, w.scan_tmp, stream);
    if (st != HTL_OK) return st;
    hipLaunchKernelGGL(k_seg_fill, dim3(grid_for(n, 256 * 4)), dim3(256), 0, stream, inverse, w.rel, n, u_max,
                       n_unique_dev, w.seg_off, w.perm);
    if (dim % 4 != 0 || dim > 1024) {
        hipLaunchKernelGGL(k_seg_elem, dim3(grid_for(u_max * dim, 256 * 4)), dim3(256), 0, stream, grad, dim, w.perm,
                           w.seg_off, u_max, n_unique_dev, out);
        return check_launch("emb_grad_segment_sum");
    }
    const int vpr = dim / 4;
    switch (team_for(vpr)) {
        case 1: launch_reduce<1, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream); break;
        case 2: launch_reduce<2, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream); break;
        case 4: launch_reduce<4, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream); break;
        case 8: launch_reduce<8, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream); break;
        case 16: launch_reduce<16, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream); break;
        case 32: launch_reduce<32, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream); break;
        default:
            if (vpr <= 64) launch_reduce<64, 1>(grad, vpr, w, u_max, n_unique_dev, out, stream);
            else if (vpr <= 128) launch_reduce<64, 2>(grad, vpr, w, u_max, n_unique_dev, out, stream);
            else launch_reduce<64, 4>(grad, vpr, w, u_max, n_unique_dev, out, stream);
            break;
    }
    return check_launch("emb_grad_segment_sum");
}

htl_status emb_rowwise_adam(htl_table* t, const int32_t* slots, const float* g, int64_t u_max,
                            const int64_t* n_unique_dev, float lr, float b1, float b2, float eps, int64_t step,
                            hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "emb_rowwise_adam: null table");
    HTL_REQUIRE(t->dev.m != nullptr && t->dtype == HTL_F32, "emb_rowwise_adam: table has no Adam state");
    HTL_REQUIRE(u_max >= 0 && u_max < ((int64_t)1 << 31), "emb_rowwise_adam: u_max out of range");
    HTL_REQUIRE(step >= 1, "emb_rowwise_adam: step must be >= 1");
    if (u_max == 0) return HTL_OK;
    HTL_REQUIRE(slots && g && aligned(slots, 4) && aligned(g, 4), "emb_rowwise_adam: null or misaligned pointer");
    const float c1 = (float)(1.0 - std::pow((double)b1, (double)step));
    const float c2 = (float)(1.0 - std::pow((double)b2, (double)step));
    const TableDev& T = t->dev;
    hipLaunchKernelGGL(k_adam, dim3(grid_for(u_max * T.dim, 256 * 4)), dim3(256), 0, stream, (float*)T.rows, T.m,
                       T.v, T.dim, T.capacity, slots, g, u_max, n_unique_dev, lr, b1, b2, eps, c1, c2);
    return check_launch("emb_rowwise_adam");
}

}  // extern "C"
