// Streaming-copy probe: the achievable HBM rate that the roofline fractions
// of the lookup kernels are read against (a measurement aid, not a step of
// the lookup path).  One 16-byte vector per thread over a full grid, the
// launch shape that copied fastest on MI355X among the ones tried (full grid
// 6.15-6.3 TB/s for 1 GiB; persistent grids of 1K-64K blocks 4.5-5.7 TB/s;
// the runtime's device-to-device copy 5.1 TB/s).
#include "htl_common.h"

namespace htl {
namespace {

constexpr int kCopyThreads = 256;
constexpr int64_t kCopyGridMax = (int64_t)1 << 22;

__global__ __launch_bounds__(kCopyThreads) void k_copy_probe(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
    for (int64_t i = blockIdx.x * (int64_t)kCopyThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" htl_status htl_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(bytes >= 0 && bytes % 16 == 0, "htl_copy_probe: bytes must be a non-negative multiple of 16");
    if (bytes == 0) return HTL_OK;
    HTL_REQUIRE(src && dst && aligned(src, 16) && aligned(dst, 16), "htl_copy_probe: null or misaligned pointer");
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_copy_probe, dim3(grid_for(n16, kCopyThreads, kCopyGridMax)), dim3(kCopyThreads), 0, stream,
                       (const u32x4*)src, (u32x4*)dst, n16);
    return check_launch("htl_copy_probe");
}
