// Device-wide exclusive prefix sum over int32 counts (reduce, scan the block
// totals, rescan with carry-in).  The length may live on the device, so
// callers need no host synchronisation for data-dependent sizes.
#include "scan.h"

namespace htl {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;
constexpr int kPerBlock = kThreads * kItems;   // 4096 values per block

__device__ __forceinline__ int64_t scan_len(int64_t n_max, const int64_t* n_dev) {
    if (!n_dev) return n_max;
    const int64_t c = *n_dev;
    return c < 0 ? 0 : (c < n_max ? c : n_max);
}

__device__ __forceinline__ int32_t xform(int32_t x, int mode, int param) {
    return mode == kScanCeilDiv ? (x + param - 1) / param : x;
}

// Block-wide exclusive scan of one value per thread; returns the block total.
__device__ int32_t block_exclusive(int32_t& v, int32_t* s_warp) {
    const int lane = __lane_id();
    const int wid = threadIdx.x >> 6;
    int32_t incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_warp[wid] = incl;
    __syncthreads();
    int32_t before = 0, total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
        const int32_t c = s_warp[w];
        if (w < wid) before += c;
        total += c;
    }
    __syncthreads();
    v = before + incl - v;
    return total;
}

__global__ __launch_bounds__(kThreads) void k_block_totals(const int32_t* __restrict__ in, int64_t n_max,
                                                          const int64_t* __restrict__ n_dev, int mode, int param,
                                                          int32_t* __restrict__ totals) {
    __shared__ int32_t s_warp[kThreads / 64];
    const int64_t n = scan_len(n_max, n_dev);
    const int64_t base = (int64_t)blockIdx.x * kPerBlock;
    int32_t sum = 0;
    for (int j = 0; j < kItems; ++j) {
        const int64_t i = base + (int64_t)j * kThreads + threadIdx.x;
        if (i < n) sum += xform(in[i], mode, param);
    }
    int32_t v = sum;
    const int32_t total = block_exclusive(v, s_warp);
    if (threadIdx.x == 0) totals[blockIdx.x] = total;
}

// One block: exclusive scan of the block totals in place.
__global__ __launch_bounds__(1024) void k_scan_totals(int32_t* __restrict__ totals, int64_t nblocks) {
    __shared__ int32_t s_warp[1024 / 64];
    __shared__ int32_t s_carry;
    if (threadIdx.x == 0) s_carry = 0;
    __syncthreads();
    for (int64_t b0 = 0; b0 < nblocks; b0 += 1024) {
        const int64_t i = b0 + threadIdx.x;
        const int32_t x = i < nblocks ? totals[i] : 0;
        const int lane = __lane_id();
        const int wid = threadIdx.x >> 6;
        int32_t incl = x;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == 63) s_warp[wid] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
        for (int w = 0; w < 1024 / 64; ++w) {
            const int32_t c = s_warp[w];
            if (w < wid) before += c;
            total += c;
        }
        const int32_t carry = s_carry;
        if (i < nblocks) totals[i] = carry + before + incl - x;
        __syncthreads();
        if (threadIdx.x == 0) s_carry = carry + total;
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void k_scan_apply(const int32_t* __restrict__ in, int64_t n_max,
                                                        const int64_t* __restrict__ n_dev, int mode, int param,
                                                        const int32_t* __restrict__ totals,
                                                        int32_t* __restrict__ out) {
    __shared__ int32_t s_warp[kThreads / 64];
    const int64_t n = scan_len(n_max, n_dev);
    const int64_t base = (int64_t)blockIdx.x * kPerBlock;
    // each thread owns kItems consecutive values
    int32_t x[kItems];
    int32_t sum = 0;
    for (int j = 0; j < kItems; ++j) {
        const int64_t i = base + (int64_t)threadIdx.x * kItems + j;
        x[j] = i < n ? xform(in[i], mode, param) : 0;
        sum += x[j];
    }
    int32_t v = sum;
    block_exclusive(v, s_warp);
    int32_t run = (totals ? totals[blockIdx.x] : 0) + v;
    for (int j = 0; j < kItems; ++j) {
        const int64_t i = base + (int64_t)threadIdx.x * kItems + j;
        if (i <= n) out[i] = run;       // out[n] receives the grand total
        run += x[j];
    }
}

}  // namespace

size_t scan_temp_bytes(int64_t n_max) { return (size_t)(ceil_div(n_max + 1, kPerBlock) + 1) * 4; }

htl_status scan_exclusive_i32(const int32_t* in, int32_t* out, int64_t n_max, const int64_t* n_dev, int mode,
                              int param, void* temp, hipStream_t s) {
    // Blocks cover indices 0..n_max inclusive so that out[n] is always written.
    const int64_t nblocks = ceil_div(n_max + 1, kPerBlock);
    if (nblocks == 1) {             // one block: no carries to compute
        hipLaunchKernelGGL(k_scan_apply, dim3(1), dim3(kThreads), 0, s, in, n_max, n_dev, mode, param,
                           (const int32_t*)nullptr, out);
        return check_launch("prefix sum");
    }
    int32_t* totals = (int32_t*)temp;
    hipLaunchKernelGGL(k_block_totals, dim3((unsigned)nblocks), dim3(kThreads), 0, s, in, n_max, n_dev, mode,
                       param, totals);
    hipLaunchKernelGGL(k_scan_totals, dim3(1), dim3(1024), 0, s, totals, nblocks);
    hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nblocks), dim3(kThreads), 0, s, in, n_max, n_dev, mode, param,
                       totals, out);
    return check_launch("prefix sum");
}

}  // namespace htl
