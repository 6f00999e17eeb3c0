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
//   (segments are laid out in a spread order q(u) = (u mod S) * C + u / S,
//   C = ceil(U / S): the dedup gives the hottest keys small, adjacent ids,
//   and their counters would otherwise share a few cache lines, so that
//   every tile's atomics queue on the same L2 channels; measured on MI355X
//   with a Zipf(1.2) batch of 2^23 IDs the count pass ran 3x slower);
//   fill   -- perm[offset[u] + place] = i (CSR of IDs grouped by unique);
//   small  -- one team of lanes per segment of <= kSmallMax IDs sums its rows;
//   large  -- longer segments (Zipf's head: the hottest key of a 2^23-ID
//             Zipf(1.2) batch owns ~18% of all rows) are cut into kChunk-row
//             chunks, one workgroup each; a one-chunk segment is finished in
//             its workgroup, the partials of longer ones are added by a
//             1024-thread workgroup per segment.
// emb_grad_segment_sum_adam runs the same passes but hands each finished
// summed row straight to Adam on the unique key's table row.
// Accumulation is fp32.  The order of IDs inside a segment depends on atomic
// order, so sums are reproducible only up to fp32 rounding.
#include <cmath>

#include "scan.h"

namespace htl {
namespace {

// Counting tile: IDs per tile and threads per block.  Its LDS (8 bytes per
// hash slot, 2 slots per ID) is 128 KB at 8192 IDs, one block per CU, so the
// block is 1024 threads to keep 16 waves per CU in flight.  On the backward
// workload (2^23 IDs, fused step): 4096 IDs x 256 threads (two blocks per
// CU) 1.640 ms; 4096 x 512 or x 1024 within noise of it; 8192 x 512
// 1.613 ms; 8192 x 1024 1.606 ms (five runs on two boxes); 8192 x 256 was
// slower (4 waves per CU).
constexpr int kCThreads = 1024;
constexpr int kCTile = 8192;
constexpr int kSmallMax = 32;              // longest segment summed by one team
constexpr int kChunk = 1024;               // rows per workgroup in long segments
constexpr int kRBlock = 256;
constexpr int kSpread = 1024;              // S of the spread segment order
constexpr int kFillUnroll = 4;             // IDs per thread and pass of the fill

// Spread order: q(u) = (u mod S) * C + u / S with C = ceil(U / S), a
// bijection from [0, U) into [0, S * C); spread_u inverts it on that range.
__device__ __forceinline__ int64_t spread_c(int64_t U) { return (U + kSpread - 1) / kSpread; }
__device__ __forceinline__ int64_t spread_q(int64_t u, int64_t C) { return (u % kSpread) * C + u / kSpread; }
__device__ __forceinline__ int64_t spread_u(int64_t q, int64_t C) { return (q % C) * kSpread + q / C; }

struct SegWs {
    int32_t* counts;       // [u_max + S], spread order
    int32_t* seg_off;      // [u_max + S + 1]
    int64_t* n_seg;        // S * C: segments in spread order
    int32_t* rel;          // [n]
    int32_t* perm;         // [n]
    int32_t* large;        // [large_max]
    int32_t* large_n;      // [large_max]: chunks of each listed segment, ceil(count / kChunk)
    int32_t* large_off;    // [large_max + 1]: chunks before each listed segment
    int32_t* part_off;     // [large_max + 1]: the same, counting multi-chunk segments only
    unsigned long long* n_large;
    void* scan_tmp;
    float* partial;        // [part_max][dim]
    int64_t large_max, max_chunks, part_max;
    size_t bytes;
};

SegWs seg_layout(int64_t n, int64_t u_max, int dim, char* base) {
    SegWs w{};
    w.large_max = n / (kSmallMax + 1) + 1;
    w.max_chunks = n / kChunk + w.large_max;
    w.part_max = 2 * (n / kChunk) + 2;     // multi-chunk segments hold > kChunk IDs each
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    const int64_t q_max = u_max + kSpread;
    w.counts = (int32_t*)take((size_t)q_max * 4);
    w.seg_off = (int32_t*)take((size_t)(q_max + 1) * 4);
    w.n_seg = (int64_t*)take(8);
    w.rel = (int32_t*)take((size_t)n * 4);
    w.perm = (int32_t*)take((size_t)n * 4);
    w.large = (int32_t*)take((size_t)w.large_max * 4);
    w.large_n = (int32_t*)take((size_t)w.large_max * 4);
    w.large_off = (int32_t*)take((size_t)(w.large_max + 1) * 4);
    w.part_off = (int32_t*)take((size_t)(w.large_max + 1) * 4);
    w.n_large = (unsigned long long*)take(8);
    w.scan_tmp = take(scan_temp_bytes(q_max));
    w.partial = (float*)take((size_t)w.part_max * dim * 4);
    w.bytes = off;
    return w;
}

__device__ __forceinline__ int64_t dev_count(int64_t n_max, const int64_t* n_dev) {
    if (!n_dev) return n_max;
    const int64_t c = *n_dev;
    return c < 0 ? 0 : (c < n_max ? c : n_max);
}

__global__ void k_seg_zero(int32_t* __restrict__ counts, int64_t u_max, const int64_t* __restrict__ n_dev,
                           unsigned long long* __restrict__ n_large, int64_t* __restrict__ n_seg) {
    const int64_t Q = kSpread * spread_c(dev_count(u_max, n_dev));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < Q; i += stride) counts[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *n_large = 0ull;
        *n_seg = Q;
    }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

// Counting tile of TILE IDs: an LDS hash of the tile's distinct uniques
// (2*TILE slots) counts each one's IDs and ranks them in tile order; then
// one atomic per (tile, unique) on the unique's counter returns the tile's
// base in the segment.  Every tile that holds a hot unique adds to that one
// counter, and those same-address atomics serialise: bigger tiles mean fewer
// of them.
template <int TILE>
__global__ __launch_bounds__(kCThreads) void k_seg_count(const int32_t* __restrict__ inverse, int64_t n,
                                                        int64_t u_max, const int64_t* __restrict__ n_dev,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ rel) {
    constexpr int CAP = 2 * TILE, CAP_LOG2 = ilog2(CAP), PER = TILE / kCThreads;
    __shared__ int32_t s_u[CAP];
    __shared__ int32_t s_cnt[CAP];          // count of each key in the tile, then its base
    const int tid = threadIdx.x;
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t C = spread_c(U);
    for (int64_t tile = blockIdx.x; tile * TILE < n; tile += gridDim.x) {
        const int64_t base = tile * TILE;
        for (int i = tid; i < CAP; i += kCThreads) {
            s_u[i] = -1;
            s_cnt[i] = 0;
        }
        __syncthreads();
        // all of the thread's inverse values are loaded before any is hashed
        // (a load in each guarded branch would wait for the one before it);
        // past the end the last ID is loaded again and ignored
        int32_t uv[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int64_t idx = base + j * kCThreads + tid;
            uv[j] = inverse[idx < n ? idx : n - 1];
        }
        int pos[PER], rank[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int64_t idx = base + j * kCThreads + tid;
            pos[j] = -1;
            rank[j] = 0;
            if (idx >= n) continue;
            const int32_t u = uv[j];
            if (u < 0 || u >= U) continue;       // outside [0, U): contributes nowhere
            const uint32_t h = (uint32_t)u * 0x9E3779B1u;
            uint32_t p = h >> (32 - CAP_LOG2);
            const uint32_t stp = ((h >> 7) | 1u) & (CAP - 1);
            for (int probe = 0; probe < CAP; ++probe) {
                const int32_t old = atomicCAS(&s_u[p], -1, u);
                if (old == -1 || old == u) break;
                p = (p + stp) & (CAP - 1);
            }
            pos[j] = (int)p;
            rank[j] = atomicAdd(&s_cnt[p], 1);
        }
        __syncthreads();
        {
            // the thread's atomics are all issued before their results are
            // stored, so they are in flight together
            constexpr int SLOTS = CAP / kCThreads;
            int32_t got[SLOTS];
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int i = k * kCThreads + tid;
                const int32_t u = s_u[i];
                got[k] = u >= 0 ? atomicAdd(&counts[spread_q(u, C)], s_cnt[i]) : 0;
            }
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int i = k * kCThreads + tid;
                if (s_u[i] >= 0) s_cnt[i] = got[k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int64_t idx = base + j * kCThreads + tid;
            if (pos[j] >= 0) rel[idx] = s_cnt[pos[j]] + rank[j];
        }
        __syncthreads();
    }
}

__global__ void k_seg_fill(const int32_t* __restrict__ inverse, const int32_t* __restrict__ rel, int64_t n,
                           int64_t u_max, const int64_t* __restrict__ n_dev, const int32_t* __restrict__ seg_off,
                           int32_t* __restrict__ perm) {
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t C = spread_c(U);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // kFillUnroll IDs per thread, each level's loads issued together (past
    // the end the last ID is loaded again and not stored)
    for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i0 < n; i0 += kFillUnroll * stride) {
        int32_t u[kFillUnroll], r[kFillUnroll], off[kFillUnroll];
#pragma unroll
        for (int k = 0; k < kFillUnroll; ++k) {
            const int64_t i = i0 + k * stride;
            const int64_t ic = i < n ? i : n - 1;
            u[k] = inverse[ic];
            r[k] = rel[ic];
        }
#pragma unroll
        for (int k = 0; k < kFillUnroll; ++k) {
            const bool ok = u[k] >= 0 && u[k] < U;
            off[k] = seg_off[spread_q(ok ? u[k] : 0, C)];
        }
#pragma unroll
        for (int k = 0; k < kFillUnroll; ++k) {
            const int64_t i = i0 + k * stride;
            if (i < n && u[k] >= 0 && u[k] < U) perm[off[k] + r[k]] = (int32_t)i;
        }
    }
}

// Adam on one element: contraction off, so every product and sum rounds on
// its own as written (the same arithmetic in every kernel that applies it).
__device__ __forceinline__ void adam_elem(float& th, float& mo, float& vo, float gj, float b1, float b2, float omb1,
                                          float omb2, float lr, float eps, float c1, float c2) {
#pragma clang fp contract(off)
    const float mj = b1 * mo + omb1 * gj;
    const float vj = b2 * vo + omb2 * (gj * gj);
    const float mhat = mj / c1;
    const float vhat = vj / c2;
    th = th - lr * (mhat / (sqrtf(vhat) + eps));
    mo = mj;
    vo = vj;
}

// Where a finished 16-byte vector v of unique u's summed gradient goes:
// into out[u] (ADAM false), or straight into Adam on the table row of
// slot[u] (ADAM true: the summed gradient is never written).
struct AdamArgs {
    float4* theta;
    float4* m;
    float4* v;
    const int32_t* slots;
    int64_t M;
    float lr, b1, b2, eps, c1, c2;
};

// Adam's state of one 16-byte vector of a row, loaded ahead of the gradient
// sum it waits for (the loads do not depend on it), then updated and stored.
struct AdamVec {
    int64_t o;      // vector index in the table's arrays; -1: not a slot of the table
    float4 th, m, v;
};

template <bool ADAM>
__device__ __forceinline__ AdamVec adam_load(int vpr, int64_t u, int v, const AdamArgs& A) {
    AdamVec r;
    r.o = -1;
    if (!ADAM) return r;
    const int32_t s = A.slots[u];
    if (s < 0 || s >= A.M) return r;
    r.o = (int64_t)s * vpr + v;
    r.th = A.theta[r.o];
    r.m = A.m[r.o];
    r.v = A.v[r.o];
    return r;
}

template <bool ADAM>
__device__ __forceinline__ void emit4(u32x4* __restrict__ out, int vpr, int64_t u, int v, float4 g,
                                      const AdamArgs& A, AdamVec st) {
    if (!ADAM) {
        u32x4 w;
        w.x = __float_as_uint(g.x);
        w.y = __float_as_uint(g.y);
        w.z = __float_as_uint(g.z);
        w.w = __float_as_uint(g.w);
        out[u * vpr + v] = w;
        return;
    }
    if (st.o < 0) return;
    const float omb1 = 1.0f - A.b1, omb2 = 1.0f - A.b2;
    adam_elem(st.th.x, st.m.x, st.v.x, g.x, A.b1, A.b2, omb1, omb2, A.lr, A.eps, A.c1, A.c2);
    adam_elem(st.th.y, st.m.y, st.v.y, g.y, A.b1, A.b2, omb1, omb2, A.lr, A.eps, A.c1, A.c2);
    adam_elem(st.th.z, st.m.z, st.v.z, g.z, A.b1, A.b2, omb1, omb2, A.lr, A.eps, A.c1, A.c2);
    adam_elem(st.th.w, st.m.w, st.v.w, g.w, A.b1, A.b2, omb1, omb2, A.lr, A.eps, A.c1, A.c2);
    A.theta[st.o] = st.th;
    A.m[st.o] = st.m;
    A.v[st.o] = st.v;
}

// Sums rows perm[beg..end) of `grad` into acc, TEAM lanes per row: team
// `team` of `teams` takes rows beg + team, beg + team + teams, ...
// Positions are 64-bit: with 32-bit ones, i0 + u * teams and the loop step
// i0 + teams * U reach end - 1 + teams * U, which passes 2^31 - 1 whenever
// end is within teams * U of it (end may be n, up to 2^31 - 1025); in 64
// bits that sum stays below 2^32.
template <int TEAM, int QMAX>
__device__ __forceinline__ void sum_rows(const u32x4* __restrict__ grad, int vpr, const int32_t* __restrict__ perm,
                                         int64_t beg, int64_t end, int team, int teams, int tl,
                                         float (&acc)[QMAX][4]) {
    constexpr int U = 4;
    for (int64_t i0 = beg + team; i0 < end; i0 += (int64_t)teams * U) {
        int32_t r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * teams;
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

// One team of TEAM lanes per segment (in spread order): most segments of a
// Zipf batch hold one to a few IDs, so a team, not a whole wavefront, takes
// each, and a wavefront keeps 64/TEAM segments' rows in flight.  Segments
// longer than kSmallMax are listed, by their spread index and chunk count,
// for the chunked path.
template <int TEAM, int QMAX, bool ADAM>
__global__ __launch_bounds__(kRBlock) void k_seg_small(const u32x4* __restrict__ grad, int vpr,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ seg_off, int64_t u_max,
                                                      const int64_t* __restrict__ n_dev, u32x4* __restrict__ out,
                                                      AdamArgs A, int32_t* __restrict__ large,
                                                      int32_t* __restrict__ large_n,
                                                      unsigned long long* __restrict__ n_large) {
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t C = spread_c(U);
    const int tl = threadIdx.x & (TEAM - 1);
    const int64_t team = (blockIdx.x * (int64_t)kRBlock + threadIdx.x) / TEAM;
    const int64_t nteams = (int64_t)gridDim.x * kRBlock / TEAM;
    for (int64_t q = team; q < kSpread * C; q += nteams) {
        const int64_t u = spread_u(q, C);
        if (u >= U) continue;                    // a hole of the spread order
        const int64_t beg = seg_off[q], end = seg_off[q + 1];
        if (end - beg > kSmallMax) {
            if (tl == 0) {
                const unsigned long long at = atomicAdd(n_large, 1ull);
                large[at] = (int32_t)q;
                large_n[at] = (int32_t)((end - beg + kChunk - 1) / kChunk);
            }
            continue;
        }
        AdamVec st[QMAX];
#pragma unroll
        for (int a = 0; a < QMAX; ++a) {
            st[a].o = -1;
            if (tl + a * TEAM < vpr) st[a] = adam_load<ADAM>(vpr, u, tl + a * TEAM, A);
        }
        float acc[QMAX][4];
#pragma unroll
        for (int a = 0; a < QMAX; ++a) acc[a][0] = acc[a][1] = acc[a][2] = acc[a][3] = 0.0f;
        sum_rows<TEAM, QMAX>(grad, vpr, perm, beg, end, 0, 1, tl, acc);
#pragma unroll
        for (int a = 0; a < QMAX; ++a) {
            const int v = tl + a * TEAM;
            if (v >= vpr) break;
            emit4<ADAM>(out, vpr, u, v, make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]), A, st[a]);
        }
    }
}

// One block: large_off = exclusive scan of the chunk counts ceil(count /
// kChunk) over the list, part_off = the same over the segments of more than
// one chunk only (a one-chunk segment's sum goes straight to the output).
// The chunk counts were listed beside the segments, so a round reads one
// coalesced array; each thread takes kLScanPer consecutive entries per round.
// On the backward workload (7,827 long segments) the scan took 29.5 us when
// it read each segment's two offsets itself (two dependent random loads per
// round of 1024 entries), 40 us with those loads issued 8 per thread at
// once (one workgroup cannot keep that many misses in flight).
constexpr int kLScanPer = 8;
__global__ __launch_bounds__(1024) void k_large_scan(const int32_t* __restrict__ large_n,
                                                    const unsigned long long* __restrict__ n_large,
                                                    int32_t* __restrict__ large_off,
                                                    int32_t* __restrict__ part_off) {
    __shared__ int32_t s_warp[16], s_warp2[16];
    __shared__ int32_t s_carry, s_carry2;
    const int64_t nl = (int64_t)*n_large;
    if (threadIdx.x == 0) s_carry = s_carry2 = 0;
    __syncthreads();
    constexpr int64_t kRound = 1024 * kLScanPer;
    for (int64_t b0 = 0; b0 <= nl; b0 += kRound) {
        const int64_t i0 = b0 + (int64_t)threadIdx.x * kLScanPer;
        int32_t x[kLScanPer];
#pragma unroll
        for (int k = 0; k < kLScanPer; ++k) x[k] = i0 + k < nl ? large_n[i0 + k] : 0;
        int32_t tot = 0, tot2 = 0;
#pragma unroll
        for (int k = 0; k < kLScanPer; ++k) {
            tot += x[k];
            tot2 += x[k] > 1 ? x[k] : 0;
        }
        const int lane = lane_id();
        const int wid = threadIdx.x >> 6;
        int32_t incl = tot, incl2 = tot2;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(incl, off);
            const int32_t y2 = __shfl_up(incl2, off);
            if (lane >= off) {
                incl += y;
                incl2 += y2;
            }
        }
        if (lane == 63) {
            s_warp[wid] = incl;
            s_warp2[wid] = incl2;
        }
        __syncthreads();
        int32_t before = 0, total = 0, before2 = 0, total2 = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wid) {
                before += s_warp[w];
                before2 += s_warp2[w];
            }
            total += s_warp[w];
            total2 += s_warp2[w];
        }
        const int32_t carry = s_carry, carry2 = s_carry2;
        int32_t run = carry + before + incl - tot, run2 = carry2 + before2 + incl2 - tot2;
#pragma unroll
        for (int k = 0; k < kLScanPer; ++k) {
            if (i0 + k <= nl) {
                large_off[i0 + k] = run;
                part_off[i0 + k] = run2;
            }
            run += x[k];
            run2 += x[k] > 1 ? x[k] : 0;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            s_carry = carry + total;
            s_carry2 = carry2 + total2;
        }
        __syncthreads();
    }
}

// One workgroup per chunk of a long segment -> partial[part_off + chunk],
// or straight to out[u] when the segment is a single chunk.
template <int TEAM, int QMAX, bool ADAM>
__global__ __launch_bounds__(kRBlock) void k_large_reduce(const u32x4* __restrict__ grad, int vpr,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ seg_off,
                                                         const int32_t* __restrict__ large,
                                                         const unsigned long long* __restrict__ n_large,
                                                         const int32_t* __restrict__ large_off,
                                                         const int32_t* __restrict__ part_off, int64_t max_chunks,
                                                         int64_t u_max, const int64_t* __restrict__ n_dev,
                                                         u32x4* __restrict__ partial, u32x4* __restrict__ out,
                                                         AdamArgs A) {
    constexpr int TEAMS = kRBlock / TEAM;
    __shared__ float s_acc[TEAMS][QMAX * TEAM * 4];
    const int64_t nl = (int64_t)*n_large;
    const int32_t total = large_off[nl];
    const int64_t C = spread_c(dev_count(u_max, n_dev));
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
        const int32_t q = large[lo];
        const int32_t part = (int32_t)(c - large_off[lo]);
        const int64_t beg = (int64_t)seg_off[q] + (int64_t)part * kChunk;
        const int64_t end = min((int64_t)seg_off[q + 1], beg + kChunk);
        const bool single = large_off[lo + 1] - large_off[lo] == 1;
        const int64_t u = spread_u(q, C);
        AdamVec st;
        st.o = -1;
        if (single && (int)threadIdx.x < vpr) st = adam_load<ADAM>(vpr, u, threadIdx.x, A);
        float acc[QMAX][4];
#pragma unroll
        for (int a = 0; a < QMAX; ++a) acc[a][0] = acc[a][1] = acc[a][2] = acc[a][3] = 0.0f;
        sum_rows<TEAM, QMAX>(grad, vpr, perm, beg, end, team, TEAMS, tl, acc);
#pragma unroll
        for (int a = 0; a < QMAX; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) s_acc[team][(a * TEAM + tl) * 4 + e] = acc[a][e];
        __syncthreads();
        u32x4* dst = partial + (int64_t)(part_off[lo] + part) * vpr;
        for (int v = threadIdx.x; v < vpr; v += kRBlock) {
            const int a = v / TEAM, l = v % TEAM;
            float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int t = 0; t < TEAMS; ++t) {
                const float* x = &s_acc[t][(a * TEAM + l) * 4];
                g.x += x[0];
                g.y += x[1];
                g.z += x[2];
                g.w += x[3];
            }
            if (single) {
                emit4<ADAM>(out, vpr, u, v, g, A, st);     // v == threadIdx.x: vpr <= kRBlock
            } else {
                u32x4 w;
                w.x = __float_as_uint(g.x);
                w.y = __float_as_uint(g.y);
                w.z = __float_as_uint(g.z);
                w.w = __float_as_uint(g.w);
                dst[v] = w;
            }
        }
        __syncthreads();
    }
}

// One workgroup per segment of several chunks: out[u] = sum of its chunk
// partials.  The
// block's kCombThreads threads are vpr-wide column lanes times groups; each
// group adds every groups-th partial (several loads in flight per thread),
// then the groups are added in LDS.  The hottest segment of a Zipf batch has
// over a thousand partials, so a serial walk over them would dominate.
constexpr int kCombThreads = 1024;

template <bool ADAM>
__global__ __launch_bounds__(kCombThreads) void k_large_combine(const u32x4* __restrict__ partial, int vpr,
                                                               int lanes, const int32_t* __restrict__ large,
                                                               const unsigned long long* __restrict__ n_large,
                                                               const int32_t* __restrict__ part_off, int64_t u_max,
                                                               const int64_t* __restrict__ n_dev,
                                                               u32x4* __restrict__ out, AdamArgs A) {
    __shared__ float4 s_red[kCombThreads];
    const int64_t nl = (int64_t)*n_large;
    const int64_t C = spread_c(dev_count(u_max, n_dev));
    const int groups = kCombThreads / lanes;
    const int l = threadIdx.x % lanes, g = threadIdx.x / lanes;
    for (int64_t i = blockIdx.x; i < nl; i += gridDim.x) {
        const int32_t c0 = part_off[i], c1 = part_off[i + 1];
        if (c1 == c0) continue;                  // a single chunk, already written
        const int64_t u = spread_u(large[i], C);
        for (int v0 = 0; v0 < vpr; v0 += lanes) {
            const int v = v0 + l;
            AdamVec st;
            st.o = -1;
            if (g == 0 && v < vpr) st = adam_load<ADAM>(vpr, u, v, A);
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            if (v < vpr) {
                constexpr int U = 4;
                int32_t c = c0 + g;
                for (; c + (U - 1) * groups < c1; c += U * groups) {
                    u32x4 x[U];
#pragma unroll
                    for (int q = 0; q < U; ++q) x[q] = partial[(int64_t)(c + q * groups) * vpr + v];
#pragma unroll
                    for (int q = 0; q < U; ++q) {
                        acc.x += __uint_as_float(x[q].x);
                        acc.y += __uint_as_float(x[q].y);
                        acc.z += __uint_as_float(x[q].z);
                        acc.w += __uint_as_float(x[q].w);
                    }
                }
                for (; c < c1; c += groups) {
                    const u32x4 x = partial[(int64_t)c * vpr + v];
                    acc.x += __uint_as_float(x.x);
                    acc.y += __uint_as_float(x.y);
                    acc.z += __uint_as_float(x.z);
                    acc.w += __uint_as_float(x.w);
                }
            }
            s_red[threadIdx.x] = acc;
            __syncthreads();
            if (g == 0 && v < vpr) {
                float4 s4 = s_red[l];
                for (int q = 1; q < groups; ++q) {
                    const float4 y = s_red[q * lanes + l];
                    s4.x += y.x;
                    s4.y += y.y;
                    s4.z += y.z;
                    s4.w += y.w;
                }
                emit4<ADAM>(out, vpr, u, v, s4, A, st);
            }
            __syncthreads();
        }
    }
}

// Element-wise fallback (dim not a multiple of 4): one thread per (u, j).
__global__ void k_seg_elem(const float* __restrict__ grad, int dim, const int32_t* __restrict__ perm,
                           const int32_t* __restrict__ seg_off, int64_t u_max, const int64_t* __restrict__ n_dev,
                           float* __restrict__ out) {
    const int64_t U = dev_count(u_max, n_dev);
    const int64_t C = spread_c(U);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < U * dim; e += stride) {
        const int64_t u = e / dim;
        const int j = (int)(e - u * dim);
        const int64_t q = spread_q(u, C);
        float s = 0.0f;
        for (int32_t i = seg_off[q]; i < seg_off[q + 1]; ++i) s += grad[(int64_t)perm[i] * dim + j];
        out[e] = s;
    }
}

int team_for(int vpr) {
    int t = 1;
    while (t < vpr && t < 64) t <<= 1;
    return t;
}

template <int TEAM, int QMAX, bool ADAM>
void launch_reduce(const float* grad, int vpr, const SegWs& w, int64_t u_max, const int64_t* n_dev, float* out,
                   const AdamArgs& A, hipStream_t s) {
    // Persistent grids: u_max bounds the segments from above (often by far:
    // 753K segments for u_max = 8.4M), and idle workgroups cost launch time.
    // Without Adam the short-segment sum is bound by the rows in flight (at
    // half its waves it took 390 against 240 us), so for rows of 16+ vectors
    // it runs half-width teams with two vectors per lane: twice the segments
    // per wave, 240 -> 222 us on the backward workload.  With Adam it is
    // bound by its bytes (half its waves: 590 -> 638 us) and keeps full teams.
    constexpr bool kHalf = !ADAM && QMAX == 1 && TEAM >= 16;
    constexpr int kSTeam = kHalf ? TEAM / 2 : TEAM, kSQmax = kHalf ? 2 : QMAX;
    hipLaunchKernelGGL((k_seg_small<kSTeam, kSQmax, ADAM>), dim3(grid_for(u_max + kSpread, kRBlock / kSTeam, 1 << 15)),
                       dim3(kRBlock), 0, s, (const u32x4*)grad, vpr, w.perm, w.seg_off, u_max, n_dev, (u32x4*)out, A,
                       w.large, w.large_n, w.n_large);
    hipLaunchKernelGGL(k_large_scan, dim3(1), dim3(1024), 0, s, w.large_n, w.n_large, w.large_off, w.part_off);
    hipLaunchKernelGGL((k_large_reduce<TEAM, QMAX, ADAM>), dim3(grid_for(w.max_chunks, 1, 1 << 14)), dim3(kRBlock),
                       0, s, (const u32x4*)grad, vpr, w.perm, w.seg_off, w.large, w.n_large, w.large_off, w.part_off,
                       w.max_chunks, u_max, n_dev, (u32x4*)w.partial, (u32x4*)out, A);
    int lanes = 1;
    while (lanes < vpr && lanes < kCombThreads / 4) lanes <<= 1;
    hipLaunchKernelGGL(k_large_combine<ADAM>, dim3(grid_for(w.large_max, 1, 1 << 14)), dim3(kCombThreads), 0, s,
                       (const u32x4*)w.partial, vpr, lanes, w.large, w.n_large, w.part_off, u_max, n_dev,
                       (u32x4*)out, A);
}

template <bool ADAM>
void launch_reduce_any(const float* grad, int vpr, const SegWs& w, int64_t u_max, const int64_t* n_dev, float* out,
                       const AdamArgs& A, hipStream_t s) {
    switch (team_for(vpr)) {
        case 1: launch_reduce<1, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s); break;
        case 2: launch_reduce<2, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s); break;
        case 4: launch_reduce<4, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s); break;
        case 8: launch_reduce<8, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s); break;
        case 16: launch_reduce<16, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s); break;
        case 32: launch_reduce<32, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s); break;
        default:
            if (vpr <= 64) launch_reduce<64, 1, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s);
            else if (vpr <= 128) launch_reduce<64, 2, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s);
            else launch_reduce<64, 4, ADAM>(grad, vpr, w, u_max, n_dev, out, A, s);
            break;
    }
}

// ---------------------------------------------------------------- Adam --
// Rows of 4k floats: TEAM lanes per row, 16 bytes per lane access.
template <int TEAM>
__global__ __launch_bounds__(256) void k_adam4(float4* __restrict__ theta, float4* __restrict__ m,
                                              float4* __restrict__ v, int vpr, int64_t M,
                                              const int32_t* __restrict__ slots, const float4* __restrict__ g,
                                              int64_t u_max, const int64_t* __restrict__ n_dev, float lr, float b1,
                                              float b2, float eps, float c1, float c2) {
    const int64_t U = dev_count(u_max, n_dev);
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    const int tl = threadIdx.x & (TEAM - 1);
    const int64_t team = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / TEAM;
    const int64_t nteams = (int64_t)gridDim.x * blockDim.x / TEAM;
    for (int64_t u = team; u < U; u += nteams) {
        const int32_t s = slots[u];
        if (s < 0 || s >= M) continue;
        for (int j = tl; j < vpr; j += TEAM) {
            const int64_t o = (int64_t)s * vpr + j;
            const float4 gj = g[u * vpr + j];
            float4 th = theta[o], mo = m[o], vo = v[o];
            adam_elem(th.x, mo.x, vo.x, gj.x, b1, b2, omb1, omb2, lr, eps, c1, c2);
            adam_elem(th.y, mo.y, vo.y, gj.y, b1, b2, omb1, omb2, lr, eps, c1, c2);
            adam_elem(th.z, mo.z, vo.z, gj.z, b1, b2, omb1, omb2, lr, eps, c1, c2);
            adam_elem(th.w, mo.w, vo.w, gj.w, b1, b2, omb1, omb2, lr, eps, c1, c2);
            theta[o] = th;
            m[o] = mo;
            v[o] = vo;
        }
    }
}

// Any dim: one thread per (u, j).
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
        adam_elem(theta[o], m[o], v[o], g[e], b1, b2, omb1, omb2, lr, eps, c1, c2);
    }
}

template <int TEAM>
void launch_adam4(const TableDev& T, const int32_t* slots, const float* g, int64_t u_max, const int64_t* n_dev,
                  float lr, float b1, float b2, float eps, float c1, float c2, hipStream_t s) {
    hipLaunchKernelGGL(k_adam4<TEAM>, dim3(grid_for(u_max, 256 / TEAM, 1 << 16)), dim3(256), 0, s, (float4*)T.rows,
                       (float4*)T.m, (float4*)T.v, T.dim / 4, T.capacity, slots, (const float4*)g, u_max, n_dev, lr,
                       b1, b2, eps, c1, c2);
}


}  // namespace
}  // namespace htl

using namespace htl;

namespace htl {
namespace {

bool fused_fallback(int dim) { return dim % 4 != 0 || dim > 1024; }

// Count, scan and fill: the CSR of IDs grouped by unique (spread order).
htl_status build_csr(const int32_t* inverse, int64_t n, const int64_t* n_dev, int64_t u_max, const SegWs& w,
                     hipStream_t stream) {
    hipLaunchKernelGGL(k_seg_zero, dim3(grid_for(u_max + kSpread, 256 * 4, 1 << 14)), dim3(256), 0, stream, w.counts,
                       u_max, n_dev, w.n_large, w.n_seg);
    hipLaunchKernelGGL(k_seg_count<kCTile>, dim3(grid_for(ceil_div(n, kCTile), 1, 1 << 16)), dim3(kCThreads), 0,
                       stream, inverse, n, u_max, n_dev, w.counts, w.rel);
    htl_status st = scan_exclusive_i32(w.counts, w.seg_off, u_max + kSpread, w.n_seg, kScanIdentity, 1, w.scan_tmp,
                                       stream);
    if (st != HTL_OK) return st;
    hipLaunchKernelGGL(k_seg_fill, dim3(grid_for(n, 256 * 4)), dim3(256), 0, stream, inverse, w.rel, n, u_max, n_dev,
                       w.seg_off, w.perm);
    return HTL_OK;
}

AdamArgs adam_args(const htl_table* t, const int32_t* slots, float lr, float b1, float b2, float eps,
                   int64_t step) {
    AdamArgs A{};
    A.theta = (float4*)t->dev.rows;
    A.m = (float4*)t->dev.m;
    A.v = (float4*)t->dev.v;
    A.slots = slots;
    A.M = t->dev.capacity;
    A.lr = lr;
    A.b1 = b1;
    A.b2 = b2;
    A.eps = eps;
    A.c1 = (float)(1.0 - std::pow((double)b1, (double)step));
    A.c2 = (float)(1.0 - std::pow((double)b2, (double)step));
    return A;
}

void launch_adam(const htl_table* t, const int32_t* slots, const float* g, int64_t u_max, const int64_t* n_dev,
                 const AdamArgs& A, hipStream_t stream) {
    const TableDev& T = t->dev;
    if (T.dim % 4 == 0 && aligned(g, 16)) {
        switch (team_for(T.dim / 4)) {
            case 1: launch_adam4<1>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
            case 2: launch_adam4<2>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
            case 4: launch_adam4<4>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
            case 8: launch_adam4<8>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
            case 16: launch_adam4<16>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
            case 32: launch_adam4<32>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
            default: launch_adam4<64>(T, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2, stream); break;
        }
    } else {
        hipLaunchKernelGGL(k_adam, dim3(grid_for(u_max * T.dim, 256 * 4)), dim3(256), 0, stream, (float*)T.rows, T.m,
                           T.v, T.dim, T.capacity, slots, g, u_max, n_dev, A.lr, A.b1, A.b2, A.eps, A.c1, A.c2);
    }
}

}  // namespace
}  // namespace htl

extern "C" {

size_t segsum_workspace_bytes(int64_t n, int64_t u_max, int dim) {
    if (n < 0) n = 0;
    if (u_max < 0) u_max = 0;
    if (dim < 1) dim = 1;
    return seg_layout(n, u_max, dim, nullptr).bytes;
}

size_t segsum_adam_workspace_bytes(int64_t n, int64_t u_max, int dim) {
    if (n < 0) n = 0;
    if (u_max < 0) u_max = 0;
    if (dim < 1) dim = 1;
    size_t b = seg_layout(n, u_max, dim, nullptr).bytes;
    if (fused_fallback(dim)) b += align_up((size_t)u_max * dim * 4, 256);
    return b;
}

htl_status emb_grad_segment_sum(const float* grad, const int32_t* inverse, int64_t n,
                                const int64_t* n_unique_dev, int64_t u_max, int dim, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31) - kSpread, "emb_grad_segment_sum: n must be in [0, 2^31 - 1024)");
    HTL_REQUIRE(u_max >= 0 && u_max <= n, "emb_grad_segment_sum: u_max must be in [0, n]");
    HTL_REQUIRE(dim >= 1 && dim <= 65536, "emb_grad_segment_sum: dim must be in [1, 65536]");
    if (n == 0 || u_max == 0) return HTL_OK;
    HTL_REQUIRE(grad && inverse && out && ws, "emb_grad_segment_sum: null pointer");
    HTL_REQUIRE(aligned(grad, 16) && aligned(out, 16) && aligned(inverse, 4) && aligned(ws, 256) &&
                    (!n_unique_dev || aligned(n_unique_dev, 8)),
                "emb_grad_segment_sum: misaligned pointer (grad/out need 16 bytes, ws 256)");
    SegWs w = seg_layout(n, u_max, dim, (char*)ws);
    HTL_REQUIRE(ws_bytes >= w.bytes, "emb_grad_segment_sum: workspace too small");
    htl_status st = build_csr(inverse, n, n_unique_dev, u_max, w, stream);
    if (st != HTL_OK) return st;
    if (fused_fallback(dim)) {
        hipLaunchKernelGGL(k_seg_elem, dim3(grid_for(u_max * dim, 256 * 4)), dim3(256), 0, stream, grad, dim, w.perm,
                           w.seg_off, u_max, n_unique_dev, out);
        return check_launch("emb_grad_segment_sum");
    }
    launch_reduce_any<false>(grad, dim / 4, w, u_max, n_unique_dev, out, AdamArgs{}, stream);
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
    launch_adam(t, slots, g, u_max, n_unique_dev, adam_args(t, slots, lr, b1, b2, eps, step), stream);
    return check_launch("emb_rowwise_adam");
}

htl_status emb_grad_segment_sum_adam(htl_table* t, const int32_t* slots, const float* grad, const int32_t* inverse,
                                     int64_t n, const int64_t* n_unique_dev, int64_t u_max, float lr, float b1,
                                     float b2, float eps, int64_t step, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(t != nullptr, "emb_grad_segment_sum_adam: null table");
    HTL_REQUIRE(t->dev.m != nullptr && t->dtype == HTL_F32, "emb_grad_segment_sum_adam: table has no Adam state");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 31) - kSpread,
                "emb_grad_segment_sum_adam: n must be in [0, 2^31 - 1024)");
    HTL_REQUIRE(u_max >= 0 && u_max <= n, "emb_grad_segment_sum_adam: u_max must be in [0, n]");
    HTL_REQUIRE(step >= 1, "emb_grad_segment_sum_adam: step must be >= 1");
    if (n == 0 || u_max == 0) return HTL_OK;
    const int dim = t->dim;
    HTL_REQUIRE(slots && grad && inverse && ws, "emb_grad_segment_sum_adam: null pointer");
    HTL_REQUIRE(aligned(grad, 16) && aligned(slots, 4) && aligned(inverse, 4) && aligned(ws, 256) &&
                    (!n_unique_dev || aligned(n_unique_dev, 8)),
                "emb_grad_segment_sum_adam: misaligned pointer (grad needs 16 bytes, ws 256)");
    SegWs w = seg_layout(n, u_max, dim, (char*)ws);
    HTL_REQUIRE(ws_bytes >= segsum_adam_workspace_bytes(n, u_max, dim),
                "emb_grad_segment_sum_adam: workspace too small");
    const AdamArgs A = adam_args(t, slots, lr, b1, b2, eps, step);
    htl_status st = build_csr(inverse, n, n_unique_dev, u_max, w, stream);
    if (st != HTL_OK) return st;
    if (fused_fallback(dim)) {
        // rows not in 16-byte vectors: the summed gradient goes through the workspace
        float* g = (float*)((char*)ws + w.bytes);
        hipLaunchKernelGGL(k_seg_elem, dim3(grid_for(u_max * dim, 256 * 4)), dim3(256), 0, stream, grad, dim, w.perm,
                           w.seg_off, u_max, n_unique_dev, g);
        launch_adam(t, slots, g, u_max, n_unique_dev, A, stream);
        return check_launch("emb_grad_segment_sum_adam");
    }
    launch_reduce_any<true>(grad, dim / 4, w, u_max, n_unique_dev, nullptr, A, stream);
    return check_launch("emb_grad_segment_sum_adam");
}

}  // extern "C"
