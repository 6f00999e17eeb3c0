// Sum-pooling of gathered rows over CSR bags (internal header): the pooled
// form of emb_gather_pool, in pool.hip.
#pragma once

#include "htl_common.h"

namespace htl {

// out[b] = sum of the rows of IDs offsets[b] .. offsets[b + 1] - 1 (fp32
// accumulation; bf16 or fp32 output), each bag clamped to the n IDs given.
// vec: a row is a whole number of 16-byte vectors, vpr of them.
htl_status launch_pooling(const TableDev& T, int dtype, bool vec, int vpr, const int32_t* slots,
                          const int32_t* inverse, int64_t n, const int32_t* offsets, int64_t nbags, bool out_bf16,
                          void* out, hipStream_t stream);

}  // namespace htl
