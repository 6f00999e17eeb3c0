// Invariant checks of a debug build (-DHTL_DEBUG); empty in release builds.
#pragma once

#include <mutex>
#include <vector>

#include "htl_common.h"

namespace htl {

// Enqueued after a find-or-insert on the same stream: slot, single copy and
// walk-length checks of every key it was given (keys, slots and status as the
// call's, n from n_dev if given).
void debug_check_foi(const TableDev& T, const int64_t* keys, int64_t n_max, const int64_t* n_dev,
                     const int32_t* slots, const uint8_t* status, hipStream_t stream);
// After a dedup: unique[inverse[i]] == keys[i], inverse[i] < n_unique <= n.
void debug_check_dedup(const int64_t* keys, int64_t n, const int64_t* unique, const int32_t* inverse,
                       const int64_t* n_unique_dev, hipStream_t stream);
// After a logged find-or-insert or erase: no live step count below zero.
void debug_check_log(const htl_table* t, hipStream_t stream);

}  // namespace htl
