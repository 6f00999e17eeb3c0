// The dedup split in two around find-or-insert (internal header), for the
// one-call forward lookup in lookup.hip.
#pragma once

#include "htl_common.h"

namespace htl {

enum { kRunDone = 0, kRunPart = 1, kRunSet = 2 };

// What the first half left for the second: which stage-2 form ran, the
// batch size and the workspace that holds the per-tile state.
struct DedupRun {
    int path;    // kRunDone: nothing left (a one-tile batch, or n == 0)
    int64_t n;
    void* ws;
    const int64_t* raw_keys;   // not null: stage 1 was skipped; the survivors are these keys
};

// First half: the unordered dedup up to unique[] and its count U (device).
// A batch of at most one tile is finished here (inverse written too).
htl_status dedup_until_unique(const char* who, const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse,
                              int64_t* n_unique_dev, void* ws, size_t ws_bytes, hipStream_t stream, DedupRun* run);

// Second half: inverse[i] and, when slots is not null, sid[i] =
// slots[inverse[i]] for every ID; slots[u] is the table slot of unique[u].
htl_status dedup_compose(const char* who, const DedupRun& run, const int32_t* slots, int32_t* inverse, int32_t* sid,
                         hipStream_t stream);

}  // namespace htl
