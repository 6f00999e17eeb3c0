// Device-wide exclusive prefix sum (segment-sum, dedup and growable-table paths).
#pragma once

#include "htl_common.h"

namespace htl {

enum { kScanIdentity = 0, kScanCeilDiv = 1 };

// out[i] = sum over j < i of f(in[j]) for i in [0, n], so out[n] is the total;
// n = min(*n_dev, n_max) when n_dev is given, else n_max.  f is the identity,
// or x -> ceil(x / param) for kScanCeilDiv.  temp: scan_temp_bytes(n_max).
size_t scan_temp_bytes(int64_t n_max);
htl_status scan_exclusive_i32(const int32_t* in, int32_t* out, int64_t n_max, const int64_t* n_dev, int mode,
                              int param, void* temp, hipStream_t s);

}  // namespace htl
