// CPU oracle for the sparse-embedding lookup path -- TEST INFRASTRUCTURE ONLY.
//
// Plain, slow, single-threaded C++17 that states what the lookup path
// computes, so the HIP library can be compared against it value by value.
// Only the test suite, the package smoke check and the benchmark's CPU
// baseline leg may load it; the HIP library never does, and the two share
// no source, header, table or constant generator.
//
// Sources:
//  * MTGenRec: An Efficient Distributed Training System for Generative
//    Recommendation Models in Meituan (arXiv 2505.12663): TL;DR and Abstract
//    (hash-based dynamic embedding table with real-time insertion/deletion,
//    automatic table merging, two-stage feature-ID deduplication), Theorem 1
//    (power-of-two table, odd probe step covers every slot), Figure 5 caption
//    (dynamic embedding table).
//  * MTGR: Industrial-Scale Generative Recommendation Framework in Meituan
//    (arXiv 2505.18654), section 5 "Training System": each key leads to its
//    embedding row and metadata; live keys are scanned compactly; IDs are
//    made unique on both sides of the all-to-all.
//  * Deep Customization of TensorFlow for Large-Scale Sparse Training at
//    Meituan, section 3.1 (hash table instead of Variables) and 3.2 (Adam).
//
// Readings where the pages are silent (each is restated in the design notes):
//  * Table contract: keys are int64; the values -1 (EMPTY) and -2 (TOMBSTONE)
//    are reserved by the table and rejected as RESERVED.  Capacity is fixed.
//  * Row initialisation: the pages give none.  A row is the closed form
//    init(key, seed) below, built from SplitMix64 outputs (Steele, Lea and
//    Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
//    Vigna's splitmix64.c), exact in fp32 and in bf16.
//  * Pooling: sum over the bag in fp64, output rounded to fp32, or from there
//    to bf16 (nearest even); an empty bag gives +0.
//  * Segment sum: fp64 accumulation (the reference value).
//  * Adam: Kingma & Ba, applied to the rows present in the batch only,
//    evaluated in fp64 and stored as fp32.
//  * Eviction: the floor(live * num / den) live keys smallest by
//    (last_seen, key), compared as (uint32, int64).
//
// Parity pins for every function live in tests/ (closed forms, brute force,
// library routines, exact arithmetic); see the docstrings there.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <cmath>
#include <numeric>
#include <unordered_map>
#include <vector>

namespace {

// ---------------------------------------------------------------- hashing --
// SplitMix64 (Steele, Lea & Flood 2014): state advances by the golden gamma,
// each output is the variant-13 finaliser of the new state.
const uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t splitmix64_next(uint64_t* state) {
    *state += kGamma;
    return mix64(*state);
}

// --------------------------------------------------------------- bfloat16 --
uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          // quiet NaN
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;                                  // round half to even
    return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// ------------------------------------------------------ closed-form rows --
// Word j of a row is half of the (j/2)-th output of a SplitMix64 stream
// seeded with base = mix64(key ^ mix64(seed)): the high half for even j, the
// low half for odd j.  fp32 element: (top 24 bits - 2^23) * 2^-26, in
// [-1/8, 1/8) with 24 significant bits, so exact.  bf16 element:
// (top 8 bits - 128) * 2^-10, at most 8 significant bits, so exact.
void init_row_f32(int64_t key, uint64_t seed, int dim, float* out) {
    uint64_t state = mix64((uint64_t)key ^ mix64(seed));
    uint64_t r = 0;
    for (int j = 0; j < dim; ++j) {
        if ((j & 1) == 0) r = splitmix64_next(&state);
        uint32_t w = (j & 1) ? (uint32_t)r : (uint32_t)(r >> 32);
        int32_t q = (int32_t)(w >> 8) - (1 << 23);
        out[j] = std::ldexp((float)q, -26);
    }
}

void init_row_bf16(int64_t key, uint64_t seed, int dim, uint16_t* out) {
    uint64_t state = mix64((uint64_t)key ^ mix64(seed));
    uint64_t r = 0;
    for (int j = 0; j < dim; ++j) {
        if ((j & 1) == 0) r = splitmix64_next(&state);
        uint32_t w = (j & 1) ? (uint32_t)r : (uint32_t)(r >> 32);
        int32_t q = (int32_t)(w >> 24) - 128;
        out[j] = f32_to_bf16_rne(std::ldexp((float)q, -10));
    }
}

// ------------------------------------------------------------ the table --
// A dynamic embedding table as an ordinary hash map: key -> entry index; the
// entries' rows live in one pooled vector.  Capacity M bounds the number of
// live keys (an open-addressing table of M slots holds at most M keys).
const int64_t kEmpty = -1;
const int64_t kTombstone = -2;

enum { ST_FOUND = 0, ST_INSERTED = 1, ST_FULL = 2, ST_RESERVED = 3 };
enum { ER_NOT_FOUND = 0, ER_ERASED = 1 };

struct Table {
    int64_t capacity;
    int dim;
    int dtype;            // 0 = fp32, 1 = bf16
    uint64_t seed;
    bool adam;
    std::unordered_map<int64_t, int64_t> index;   // key -> entry
    std::vector<int64_t> free_entries;
    std::vector<float> rows_f32;
    std::vector<uint16_t> rows_bf16;
    std::vector<uint32_t> last_seen;
    std::vector<float> m, v;

    int64_t new_entry(int64_t key) {
        int64_t e;
        if (!free_entries.empty()) {
            e = free_entries.back();
            free_entries.pop_back();
        } else {
            e = (int64_t)last_seen.size();
            last_seen.push_back(0);
            if (dtype == 0) rows_f32.resize(rows_f32.size() + dim);
            else rows_bf16.resize(rows_bf16.size() + dim);
            if (adam) { m.resize(m.size() + dim); v.resize(v.size() + dim); }
        }
        if (dtype == 0) init_row_f32(key, seed, dim, &rows_f32[e * dim]);
        else init_row_bf16(key, seed, dim, &rows_bf16[e * dim]);
        if (adam) {
            std::fill(m.begin() + e * dim, m.begin() + (e + 1) * dim, 0.0f);
            std::fill(v.begin() + e * dim, v.begin() + (e + 1) * dim, 0.0f);
        }
        return e;
    }

    float elem(int64_t e, int j) const {
        return dtype == 0 ? rows_f32[e * dim + j] : bf16_to_f32(rows_bf16[e * dim + j]);
    }
};

}  // namespace

extern "C" {

// ----------------------------------------------------------- primitives --
uint64_t orc_mix64(uint64_t x) { return mix64(x); }

void orc_splitmix64(uint64_t seed, int64_t n, uint64_t* out) {
    uint64_t s = seed;
    for (int64_t i = 0; i < n; ++i) out[i] = splitmix64_next(&s);
}

uint16_t orc_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

// Closed-form initial row of `key` (dtype 0: float[dim]; 1: bf16 bits[dim]).
void orc_init_row(int64_t key, uint64_t seed, int32_t dim, int32_t dtype, void* out) {
    if (dtype == 0) init_row_f32(key, seed, dim, (float*)out);
    else init_row_bf16(key, seed, dim, (uint16_t*)out);
}

// ------------------------------------------------------------ Theorem 1 --
// MTGenRec, Theorem 1: for M = 2^n and the probe sequence
// h_t = (h0 + t*S) mod M, t = 0..M-1, count the distinct slots visited.
int64_t orc_probe_coverage(uint64_t M, uint64_t h0, uint64_t S) {
    std::vector<char> seen(M, 0);
    int64_t count = 0;
    uint64_t h = h0 % M;
    uint64_t step = S % M;
    for (uint64_t t = 0; t < M; ++t) {
        if (!seen[h]) { seen[h] = 1; ++count; }
        h = (h + step) % M;
    }
    return count;
}

// Bucketed form: M slots in M/W buckets of W consecutive slots; the probe
// walks buckets b_t = (b0 + t*S) mod (M/W), t = 0..M/W-1, and every visited
// bucket contributes all W of its slots.  Returns the distinct slots covered.
int64_t orc_bucket_probe_coverage(uint64_t M, uint64_t W, uint64_t b0, uint64_t S) {
    uint64_t nb = M / W;
    std::vector<char> seen(M, 0);
    int64_t count = 0;
    uint64_t b = b0 % nb;
    uint64_t step = S % nb;
    for (uint64_t t = 0; t < nb; ++t) {
        for (uint64_t w = 0; w < W; ++w) {
            uint64_t slot = b * W + w;
            if (!seen[slot]) { seen[slot] = 1; ++count; }
        }
        b = (b + step) % nb;
    }
    return count;
}

// ---------------------------------------------------------------- dedup --
// Feature-ID deduplication (MTGenRec TL;DR, "two-stage ID deduplication";
// MTGR section 5 "Embedding Lookup").  Both stages together compute the
// plain unique-with-inverse: unique = sorted distinct keys,
// inverse[i] = position of keys[i] in unique.  Returns U.
int64_t orc_dedup(const int64_t* keys, int64_t n, int64_t* unique, int32_t* inverse) {
    std::vector<int64_t> u(keys, keys + n);
    std::sort(u.begin(), u.end());
    u.erase(std::unique(u.begin(), u.end()), u.end());
    for (int64_t i = 0; i < n; ++i)
        inverse[i] = (int32_t)(std::lower_bound(u.begin(), u.end(), keys[i]) - u.begin());
    std::copy(u.begin(), u.end(), unique);
    return (int64_t)u.size();
}

// ---------------------------------------------------------------- table --
void* orc_table_create(int64_t capacity, int32_t dim, int32_t dtype, uint64_t seed,
                       int32_t with_adam) {
    Table* t = new Table();
    t->capacity = capacity;
    t->dim = dim;
    t->dtype = dtype;
    t->seed = seed;
    t->adam = with_adam != 0;
    return t;
}

void orc_table_destroy(void* h) { delete (Table*)h; }

int64_t orc_table_size(void* h) { return (int64_t)((Table*)h)->index.size(); }

// Capacity expansion (MTGR section 5: capacity grows while keys keep their
// vectors and metadata).  The map holds no slots, so growing is a change of
// the bound that makes a table FULL; every live key keeps its row, last_seen
// and Adam state.  Returns 0 if the new capacity is below the live count.
int32_t orc_table_resize(void* h, int64_t capacity) {
    Table* t = (Table*)h;
    if (capacity < (int64_t)t->index.size()) return 0;
    t->capacity = capacity;
    return 1;
}

// Find-or-insert (MTGenRec abstract: real-time insertion into a dynamic hash
// table; MTGR section 5: keys map to vectors and metadata).  Keys are taken
// in call order: a reserved key is RESERVED; a present key is FOUND; with M
// live keys the table is FULL; otherwise the key is INSERTED with its
// closed-form initial row (and zero Adam state).  FOUND and INSERTED keys
// get last_seen = step.
void orc_find_or_insert(void* h, const int64_t* keys, int64_t n, uint32_t step,
                        uint8_t* status) {
    Table* t = (Table*)h;
    for (int64_t i = 0; i < n; ++i) {
        int64_t k = keys[i];
        if (k == kEmpty || k == kTombstone) { status[i] = ST_RESERVED; continue; }
        auto it = t->index.find(k);
        if (it != t->index.end()) {
            t->last_seen[it->second] = step;
            status[i] = ST_FOUND;
            continue;
        }
        if ((int64_t)t->index.size() >= t->capacity) { status[i] = ST_FULL; continue; }
        int64_t e = t->new_entry(k);
        t->last_seen[e] = step;
        t->index.emplace(k, e);
        status[i] = ST_INSERTED;
    }
}

// Delete (MTGenRec abstract: real-time deletion).  ERASED if the key was
// live, NOT_FOUND otherwise (reserved values are never live).
void orc_erase(void* h, const int64_t* keys, int64_t n, uint8_t* status) {
    Table* t = (Table*)h;
    for (int64_t i = 0; i < n; ++i) {
        auto it = t->index.find(keys[i]);
        if (it == t->index.end()) { status[i] = ER_NOT_FOUND; continue; }
        t->free_entries.push_back(it->second);
        t->index.erase(it);
        status[i] = ER_ERASED;
    }
}

// Read one entry.  Returns 1 and fills the outputs (any may be null) if the
// key is live, else 0.  row_out is float[dim] or bf16 bits[dim] by dtype.
int32_t orc_lookup(void* h, int64_t key, void* row_out, uint32_t* last_seen_out,
                   float* m_out, float* v_out) {
    Table* t = (Table*)h;
    auto it = t->index.find(key);
    if (it == t->index.end()) return 0;
    int64_t e = it->second;
    if (row_out) {
        if (t->dtype == 0) std::memcpy(row_out, &t->rows_f32[e * t->dim], sizeof(float) * t->dim);
        else std::memcpy(row_out, &t->rows_bf16[e * t->dim], sizeof(uint16_t) * t->dim);
    }
    if (last_seen_out) *last_seen_out = t->last_seen[e];
    if (t->adam && m_out) std::memcpy(m_out, &t->m[e * t->dim], sizeof(float) * t->dim);
    if (t->adam && v_out) std::memcpy(v_out, &t->v[e * t->dim], sizeof(float) * t->dim);
    return 1;
}

// Row gather: out[i] = row(keys[i]), a copy in the table dtype; a key that is
// not live gives a zero row.
void orc_gather(void* h, const int64_t* keys, int64_t n, void* out) {
    Table* t = (Table*)h;
    size_t esz = t->dtype == 0 ? 4 : 2;
    char* o = (char*)out;
    for (int64_t i = 0; i < n; ++i) {
        auto it = t->index.find(keys[i]);
        char* dst = o + (size_t)i * t->dim * esz;
        if (it == t->index.end()) { std::memset(dst, 0, t->dim * esz); continue; }
        const void* src = t->dtype == 0 ? (const void*)&t->rows_f32[it->second * t->dim]
                                        : (const void*)&t->rows_bf16[it->second * t->dim];
        std::memcpy(dst, src, t->dim * esz);
    }
}

// Sum pooling over multi-hot bags: pooled[b] = sum of row(keys[i]) for i in
// [offsets[b], offsets[b+1]), accumulated in fp64; keys that are not live add
// nothing; an empty bag gives +0.  out_dtype 0 writes the fp64 sum rounded to
// fp32; 1 writes that fp32 value rounded to bf16 (nearest even).  For bf16
// rows every partial sum is exact in fp32 (see the tests), so the result does
// not depend on the order of accumulation.
void orc_gather_pool(void* h, const int64_t* keys, const int32_t* offsets, int64_t nbags,
                     int32_t out_dtype, void* out) {
    Table* t = (Table*)h;
    std::vector<double> acc(t->dim);
    for (int64_t b = 0; b < nbags; ++b) {
        std::fill(acc.begin(), acc.end(), 0.0);
        for (int64_t i = offsets[b]; i < offsets[b + 1]; ++i) {
            auto it = t->index.find(keys[i]);
            if (it == t->index.end()) continue;
            for (int j = 0; j < t->dim; ++j) acc[j] += (double)t->elem(it->second, j);
        }
        for (int j = 0; j < t->dim; ++j) {
            const float s = (float)acc[j];
            if (out_dtype == 0) ((float*)out)[b * t->dim + j] = s;
            else ((uint16_t*)out)[b * t->dim + j] = f32_to_bf16_rne(s);
        }
    }
}

// Backward gradient dedup + segment sum: sum[u] = sum of grad[i] over
// inverse[i] == u, in fp64; abs_sum[u] = sum of |grad[i]| (the scale of the
// summation error bound).  Either output may be null.
void orc_segment_sum(const float* grad, const int32_t* inverse, int64_t n, int64_t n_unique,
                     int32_t dim, double* sum_out, double* abs_out) {
    if (sum_out) std::fill(sum_out, sum_out + n_unique * dim, 0.0);
    if (abs_out) std::fill(abs_out, abs_out + n_unique * dim, 0.0);
    for (int64_t i = 0; i < n; ++i) {
        int64_t u = inverse[i];
        for (int j = 0; j < dim; ++j) {
            double g = (double)grad[i * dim + j];
            if (sum_out) sum_out[u * dim + j] += g;
            if (abs_out) abs_out[u * dim + j] += std::fabs(g);
        }
    }
}

// Row-wise Adam (Kingma & Ba, Algorithm 1), one element, step t >= 1,
// evaluated in fp64 from the fp32 state:
//   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g^2;
//   theta = theta - lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps),
// then theta, m and v are stored back rounded to fp32.
static void adam_elem(float& th, float& mj, float& vj, float g, double lr, double b1, double b2,
                      double eps, double c1, double c2) {
    const double gj = g;
    const double m2 = b1 * (double)mj + (1.0 - b1) * gj;
    const double v2 = b2 * (double)vj + (1.0 - b2) * gj * gj;
    const double upd = (m2 / c1) / (std::sqrt(v2 / c2) + eps);
    th = (float)((double)th - lr * upd);
    mj = (float)m2;
    vj = (float)v2;
}

// Adam over the rows of the given (distinct) keys: only those rows change
// (lazy update); keys that are not live are skipped.  Requires an fp32 table
// created with Adam state.
void orc_adam(void* h, const int64_t* keys, const float* g, int64_t n, float lr, float b1,
              float b2, float eps, int64_t step) {
    Table* t = (Table*)h;
    if (!t->adam || t->dtype != 0) return;
    const double c1 = 1.0 - std::pow((double)b1, (double)step);
    const double c2 = 1.0 - std::pow((double)b2, (double)step);
    for (int64_t i = 0; i < n; ++i) {
        auto it = t->index.find(keys[i]);
        if (it == t->index.end()) continue;
        int64_t e = it->second;
        for (int j = 0; j < t->dim; ++j)
            adam_elem(t->rows_f32[e * t->dim + j], t->m[e * t->dim + j], t->v[e * t->dim + j],
                      g[i * t->dim + j], lr, b1, b2, eps, c1, c2);
    }
}

// The same update on plain arrays of n elements (theta, m, v updated in place).
void orc_adam_arrays(float* theta, float* m, float* v, const float* g, int64_t n, float lr,
                     float b1, float b2, float eps, int64_t step) {
    const double c1 = 1.0 - std::pow((double)b1, (double)step);
    const double c2 = 1.0 - std::pow((double)b2, (double)step);
    for (int64_t i = 0; i < n; ++i)
        adam_elem(theta[i], m[i], v[i], g[i], lr, b1, b2, eps, c1, c2);
}

// Adam in single precision, every operation rounded to fp32 as written (no
// fused multiply-add: the oracle is built with -ffp-contract=off), in the
// order of Kingma & Ba's Algorithm 1 for a table kept in fp32 (the
// TensorFlow article, section 3.2, keeps Adam's bias terms per server; here
// they are per-call scalars):
//   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g);
//   theta = theta - lr * ((m / c1) / (sqrt(v / c2) + eps)),
// with 1-b1, 1-b2 in fp32 and c1 = 1-b1^t, c2 = 1-b2^t formed in fp64 and
// rounded to fp32.  sqrtf and fp32 division are correctly rounded (IEEE
// 754), so this is one determined value per element.
void orc_adam_arrays_f32(float* theta, float* m, float* v, const float* g, int64_t n, float lr,
                         float b1, float b2, float eps, int64_t step) {
    const float c1 = (float)(1.0 - std::pow((double)b1, (double)step));
    const float c2 = (float)(1.0 - std::pow((double)b2, (double)step));
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    for (int64_t i = 0; i < n; ++i) {
        const float gi = g[i];
        const float mi = b1 * m[i] + omb1 * gi;
        const float vi = b2 * v[i] + omb2 * (gi * gi);
        const float mh = mi / c1;
        const float vh = vi / c2;
        theta[i] = theta[i] - lr * (mh / (std::sqrt(vh) + eps));
        m[i] = mi;
        v[i] = vi;
    }
}

// Live keys with their last_seen (MTGR section 5, compact key scanning), in
// ascending key order.  Returns the live count; outputs may be null.
int64_t orc_live(void* h, int64_t* keys_out, uint32_t* last_seen_out) {
    Table* t = (Table*)h;
    std::vector<std::pair<int64_t, int64_t>> kv(t->index.begin(), t->index.end());
    std::sort(kv.begin(), kv.end());
    for (size_t i = 0; i < kv.size(); ++i) {
        if (keys_out) keys_out[i] = kv[i].first;
        if (last_seen_out) last_seen_out[i] = t->last_seen[kv[i].second];
    }
    return (int64_t)kv.size();
}

// Least-recently-used victims: k = floor(live * num / den) live keys, the
// smallest by (last_seen, key).  Writes them in that order; returns k.
int64_t orc_lru_victims(void* h, int64_t num, int64_t den, int64_t* victims_out) {
    Table* t = (Table*)h;
    std::vector<std::pair<uint32_t, int64_t>> order;
    order.reserve(t->index.size());
    for (const auto& kv : t->index) order.emplace_back(t->last_seen[kv.second], kv.first);
    std::sort(order.begin(), order.end());
    int64_t k = (int64_t)((__int128)order.size() * num / den);
    for (int64_t i = 0; i < k; ++i) victims_out[i] = order[i].second;
    return k;
}

}  // extern "C"
