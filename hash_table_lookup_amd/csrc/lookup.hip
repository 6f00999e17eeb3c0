// The forward lookup in one call: dedup -> find-or-insert -> gather (or
// bag sum-pooling), with the same results as the three calls.
//
// MTGenRec (arXiv 2505.12663), TL;DR and Figure 5: IDs are deduplicated in
// two stages, then looked up in the dynamic hash table; MTGR (arXiv
// 2505.18654) section 5, "Embedding Lookup" and "Other Optimizations": the
// lookup of a batch's deduplicated IDs is one stage of the training step.
//
// What the single call changes is the order of the dedup's last pass.  The
// three calls compose inverse[i] per tile of IDs in the dedup, and the
// gather then reads, per ID, inverse[i] and slots[inverse[i]] -- a random
// 4-byte load that every row read waits for.  Here the per-tile compose runs
// after find-or-insert: each tile survivor fetches its key's slot once into
// LDS, and the pass writes both inverse[i] and sid[i] = slots[inverse[i]].
// The gather then walks sid in sequence (one dependent load per row, not
// two), and the random slot loads drop from one per ID to one per tile
// survivor.
#include "debug.h"
#include "lookup.h"

namespace htl {
namespace {

size_t sid_offset(int64_t n) { return align_up(dedup_workspace_bytes(n), 256); }

// id_slots[i] = slots[inverse[i]] (batches that the dedup finished in one
// tile, where no per-tile compose is left to write it).
__global__ void k_id_slots(const int32_t* __restrict__ slots, const int32_t* __restrict__ inverse, int64_t n,
                           int32_t* __restrict__ id_slots) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        id_slots[i] = slots[inverse[i]];
}

}  // namespace
}  // namespace htl

using namespace htl;

extern "C" {

htl_status emb_lookup_slots(htl_table* t, const int64_t* keys, int64_t n, uint32_t step, int64_t* unique,
                            int32_t* inverse, int64_t* n_unique_dev, int32_t* slots, uint8_t* status,
                            int32_t* id_slots, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    // every argument is checked before the first launch
    HTL_REQUIRE(t != nullptr, "emb_lookup_slots: null table");
    HTL_REQUIRE(n >= 0 && n < ((int64_t)1 << 30), "emb_lookup_slots: n must be in [0, 2^30)");
    HTL_REQUIRE(n_unique_dev && aligned(n_unique_dev, 8), "emb_lookup_slots: null or misaligned n_unique_dev");
    HTL_REQUIRE(!t->dev.last_seen || step != kLsDead,
                "emb_lookup_slots: step 0xFFFFFFFF is reserved on a table that keeps last_seen");
    if (n > 0) {
        HTL_REQUIRE(keys && unique && inverse && slots && status && id_slots && ws, "emb_lookup_slots: null pointer");
        HTL_REQUIRE(aligned(keys, 8) && aligned(unique, 8) && aligned(inverse, 4) && aligned(slots, 4) &&
                        aligned(id_slots, 4) && aligned(ws, 256),
                    "emb_lookup_slots: misaligned pointer");
        HTL_REQUIRE(ws_bytes >= dedup_workspace_bytes(n), "emb_lookup_slots: workspace too small");
    }
    DedupRun run{kRunDone, n, ws};
    htl_status st = dedup_until_unique("emb_lookup_slots", keys, n, unique, inverse, n_unique_dev, ws, ws_bytes,
                                       stream, &run);
    if (st != HTL_OK) return st;
    st = ht_find_or_insert(t, unique, n, n_unique_dev, step, slots, status, stream);
    if (st != HTL_OK) return st;
    if (n == 0) return HTL_OK;
    if (run.path == kRunDone) {   // one tile: the dedup wrote the inverse already
        hipLaunchKernelGGL(k_id_slots, dim3(grid_for(n, 256)), dim3(256), 0, stream, slots, inverse, n, id_slots);
        st = check_launch("emb_lookup_slots");
    } else {
        st = dedup_compose("emb_lookup_slots", run, slots, inverse, id_slots, stream);
    }
    if (st == HTL_OK) debug_check_dedup(keys, n, unique, inverse, n_unique_dev, stream);
    return st;
}

size_t emb_lookup_workspace_bytes(int64_t n) {
    if (n < 0) n = 0;
    return sid_offset(n) + align_up((size_t)(n > 0 ? n : 1) * 4, 256);
}

htl_status emb_lookup(htl_table* t, const int64_t* keys, int64_t n, uint32_t step, int64_t* unique,
                      int32_t* inverse, int64_t* n_unique_dev, int32_t* slots, uint8_t* status,
                      const int32_t* offsets, int64_t nbags, htl_dtype out_dtype, void* out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
    clear_error();
    // the gather's arguments are checked before the first launch too
    HTL_REQUIRE(t != nullptr, "emb_lookup: null table");
    HTL_REQUIRE(out_dtype == HTL_F32 || out_dtype == HTL_BF16, "emb_lookup: bad out_dtype");
    if (offsets == nullptr)
        HTL_REQUIRE(out_dtype == t->dtype || (t->dtype == HTL_BF16 && out_dtype == HTL_F32),
                    "emb_lookup: without pooling out_dtype must be the table dtype or fp32");
    else
        HTL_REQUIRE(nbags >= 0 && nbags < ((int64_t)1 << 31) && aligned(offsets, 4),
                    "emb_lookup: nbags out of range or misaligned offsets");
    const bool any_out = offsets ? nbags > 0 : n > 0;
    HTL_REQUIRE(!any_out || (out && aligned(out, 16)), "emb_lookup: null or misaligned out (16 bytes)");
    HTL_REQUIRE(n <= 0 || ws_bytes >= emb_lookup_workspace_bytes(n), "emb_lookup: workspace too small");
    int32_t* sid = n > 0 && ws ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + sid_offset(n)) : nullptr;
    htl_status st = emb_lookup_slots(t, keys, n, step, unique, inverse, n_unique_dev, slots, status, sid, ws,
                                     n > 0 ? sid_offset(n) : ws_bytes, stream);
    if (st != HTL_OK) return st;
    return emb_gather_pool(t, sid, nullptr, n, offsets, nbags, out_dtype, out, stream);
}

}  // extern "C"
