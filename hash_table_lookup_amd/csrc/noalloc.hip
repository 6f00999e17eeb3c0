// dedup_unique_inverse for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same kernels as dedup_unique_inverse, with the workspace
// taken from a fixed array in device memory that the library's code object
// carries.
//
// The array is a file-scope __device__ variable.  On the host its name is a
// host-side stand-in, not a device address, so it is never passed to a
// kernel or a copy: the first call on each device (with that device
// current) looks up the device address with hipGetSymbolAddress and keeps it
// per device, and every later call on that device passes that address.  Each
// device holds its own copy of the array, from the first use of the library
// on it until the process ends.
#include <mutex>

#include "htl_common.h"

namespace htl {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per device
constexpr int64_t kNoAllocMaxKeys = (int64_t)1 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's copy of `scratch` (looked up once).
htl_status scratch_address(const char* who, void** out) {
    int dev = -1;
    HTL_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(HTL_ERR_DEVICE, std::string(who) + ": device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(HTL_ERR_DEVICE, std::string(who) + ": hipGetSymbolAddress of the scratch array failed: " +
                                            hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return HTL_OK;
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

int64_t dedup_noalloc_max_keys(void) { return kNoAllocMaxKeys; }

htl_status dedup_unique_inverse_noalloc(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                                        int64_t* n_unique_dev, hipStream_t stream) {
    clear_error();
    HTL_REQUIRE(n >= 0 && n <= kNoAllocMaxKeys,
                "dedup_unique_inverse_noalloc: n must be in [0, 2^20] (the static scratch holds the workspace of "
                "at most 2^20 keys)");
    const size_t need = dedup_workspace_bytes(n);
    HTL_REQUIRE(need <= kScratchBytes, "dedup_unique_inverse_noalloc: workspace exceeds the static scratch");
    void* ws = nullptr;
    const htl_status st = scratch_address("dedup_unique_inverse_noalloc", &ws);
    if (st != HTL_OK) return st;
    return dedup_unique_inverse(keys, n, unique, inverse, n_unique_dev, ws, kScratchBytes, stream);
}

}  // extern "C"
