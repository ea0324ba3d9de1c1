// Host side of libgr: argument validation, the GTM SID trie builder
// (GRACE Section 4.4 and Appendix A: CSR trie, subtree-union matchers of
// eqs 4 and 9, deduplicated matcher tables), trie upload, request-side Bloom
// probe encoding (Section 4.3) and the dispatch of the hot-path kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "gr_internal.h"

using namespace gr;

namespace {

thread_local std::string g_err;

gr_status fail(gr_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

gr_status hip_fail(hipError_t e, const char *what) {
    return fail(GR_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

gr_status gr::report(gr_status st, const char *msg) { return fail(st, "%s", msg); }

namespace {

int hw_threads(int req) {
    if (req > 0) return req;
    unsigned n = std::thread::hardware_concurrency();
    return n ? (int)std::min(n, 64u) : 4;
}

template <typename F>
void parallel_for(int64_t n, int threads, F f) {
    if (n <= 0) return;
    threads = (int)std::max<int64_t>(1, std::min<int64_t>(threads, n / 4096 + 1));
    if (threads == 1) { f(0, n); return; }
    std::vector<std::thread> th;
    int64_t chunk = (n + threads - 1) / threads;
    for (int i = 0; i < threads; ++i) {
        int64_t a = i * chunk, b = std::min(n, a + chunk);
        if (a >= b) break;
        th.emplace_back([=] { f(a, b); });
    }
    for (auto &t : th) t.join();
}

// Bloom positions of one id: first SplitMix64 output from state `id`
// (Steele, Lea and Flood 2014), split into h1 (low half) and h2 (high half
// forced odd), position i = (h1 + i*h2) mod w (Kirsch and Mitzenmacher 2006).
inline void bloom_pos(uint64_t id, uint32_t w_bits, int k, uint32_t *out) {
    uint64_t z = id + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    uint32_t h1 = (uint32_t)z, h2 = (uint32_t)(z >> 32) | 1u;
    for (int i = 0; i < k; ++i) out[i] = (h1 + (uint32_t)i * h2) & (w_bits - 1u);
}

inline uint64_t row_hash(const uint64_t *r, int w) {
    uint64_t h = 0x2545F4914F6CDD1Dull ^ (uint64_t)w;
    for (int i = 0; i < w; ++i) {
        h ^= r[i] + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
        h *= 0xFF51AFD7ED558CCDull;
    }
    return h ^ (h >> 33);
}

// Deduplicated table of fixed-width rows (open addressing on a row hash,
// collisions resolved by comparing whole rows).
struct RowTable {
    int w = 0;
    std::vector<uint64_t> rows;   // [n, w]
    int64_t n = 0;
    std::vector<int32_t> slot;
    uint64_t mask = 0;

    void init(int width, int64_t expected) {
        w = width;
        n = 0;
        uint64_t cap = 16;
        while (cap < (uint64_t)(expected * 2 + 16)) cap <<= 1;
        slot.assign(cap, -1);
        mask = cap - 1;
    }
    void grow() {
        std::vector<int32_t> old(slot.size() * 2, -1);
        slot.swap(old);
        mask = slot.size() - 1;
        for (int64_t i = 0; i < n; ++i) place(i, row_hash(&rows[i * w], w));
    }
    void place(int64_t id, uint64_t h) {
        uint64_t s = h & mask;
        while (slot[s] >= 0) s = (s + 1) & mask;
        slot[s] = (int32_t)id;
    }
    // Returns the id of `r` (inserting it if new).  `r` may alias the slot
    // rows[n*w] (in-place compaction of an already filled buffer).
    int32_t insert(const uint64_t *r) {
        if ((uint64_t)(n * 2 + 2) > slot.size()) grow();
        uint64_t h = row_hash(r, w), s = h & mask;
        while (slot[s] >= 0) {
            const uint64_t *o = &rows[(int64_t)slot[s] * w];
            if (std::memcmp(o, r, sizeof(uint64_t) * w) == 0) return slot[s];
            s = (s + 1) & mask;
        }
        int64_t id = n++;
        uint64_t *dst = &rows[id * w];
        if (dst != r) std::memmove(dst, r, sizeof(uint64_t) * w);
        slot[s] = (int32_t)id;
        return (int32_t)id;
    }
};

template <typename T>
hipError_t upload(T **dptr, const T *src, size_t n) {
    *dptr = nullptr;
    if (n == 0) return hipSuccess;
    hipError_t e = hipMalloc((void **)dptr, n * sizeof(T));
    if (e != hipSuccess) return e;
    return hipMemcpy(*dptr, src, n * sizeof(T), hipMemcpyHostToDevice);
}

}  // namespace

// ---------------------------------------------------------------------------
// Opaque handles
// ---------------------------------------------------------------------------

struct gr_trie_builder {
    gr_trie_params p{};
    int w_bl = 0, bpt = 0, threads = 1;
    int64_t n_in = 0, n_leaf = 0;
    std::vector<int64_t> leaf_of_input;  // input row -> leaf index
    std::vector<uint64_t> leaf_key;      // sorted distinct packed SIDs
    std::vector<int64_t> n_level;        // nodes per level 0..L
    std::vector<int64_t> n_multi;        // nodes with >= 2 children per level
    std::vector<uint64_t> leaf_bm;       // [n_leaf (+ room), w_bm]
    std::vector<uint64_t> leaf_bl;       // [n_leaf (+ room), w_bl]
};

struct gr_trie {
    TrieDev d{};
    int device = 0;
    bool has_host = false;
    std::vector<int32_t> h_off, h_child, h_bmi, h_bli, h_depth, h_parent;
    std::vector<int16_t> h_tok, h_ntok;
    std::vector<uint64_t> h_bm, h_bl;
    std::vector<int32_t> h_kw_off, h_kw_bmi, h_kw_bli;
    bool host_only = false;
};

extern "C" {

const char *gr_last_error(void) { return g_err.c_str(); }
const char *gr_version(void) { return "libgr 0.1 (gfx950)"; }

gr_status gr_bloom_probes(const int32_t *ids, int64_t n, int32_t bloom_bits,
                          int32_t bloom_k, uint32_t *positions) {
    if (n < 0 || (n > 0 && (!ids || !positions)))
        return fail(GR_E_INVALID, "gr_bloom_probes: null array");
    if (bloom_bits < 64 || bloom_bits > 65536 || (bloom_bits & (bloom_bits - 1)))
        return fail(GR_E_INVALID, "gr_bloom_probes: bloom_bits %d is not a power of two in [64, 65536]", bloom_bits);
    if (bloom_k < 1 || bloom_k > 16)
        return fail(GR_E_INVALID, "gr_bloom_probes: bloom_k %d not in [1, 16]", bloom_k);
    for (int64_t i = 0; i < n; ++i) {
        if (ids[i] < 0) return fail(GR_E_INVALID, "gr_bloom_probes: id[%lld] < 0", (long long)i);
        bloom_pos((uint64_t)ids[i], (uint32_t)bloom_bits, bloom_k, positions + i * bloom_k);
    }
    return GR_OK;
}

// ---------------------------------------------------------------------------
// Trie builder
// ---------------------------------------------------------------------------

gr_status gr_trie_builder_create(const gr_trie_params *params, const int32_t *sids,
                                 int64_t n_sids, gr_trie_builder **out) {
    if (!params || !out || (n_sids > 0 && !sids))
        return fail(GR_E_INVALID, "gr_trie_builder_create: null argument");
    *out = nullptr;
    const gr_trie_params &p = *params;
    if (p.sid_length < 1 || p.sid_length > 16)
        return fail(GR_E_INVALID, "sid_length %d not in [1, 16]", p.sid_length);
    if (p.vocab_size < 2 || p.vocab_size > 32768)
        return fail(GR_E_INVALID, "vocab_size %d not in [2, 32768]", p.vocab_size);
    if (p.w_bm < 1 || p.w_bm > MAX_WBM)
        return fail(GR_E_INVALID, "w_bm %d not in [1, %d]", p.w_bm, MAX_WBM);
    if (p.bloom_bits != 0) {
        if (p.bloom_bits < 64 || p.bloom_bits > 65536 || (p.bloom_bits & (p.bloom_bits - 1)))
            return fail(GR_E_INVALID, "bloom_bits %d is not 0 or a power of two in [64, 65536]", p.bloom_bits);
        if (p.bloom_k < 1 || p.bloom_k > 16)
            return fail(GR_E_INVALID, "bloom_k %d not in [1, 16]", p.bloom_k);
    }
    if (p.bloom_slice_min < -1)
        return fail(GR_E_INVALID, "bloom_slice_min %d is not -1, 0 or a child count", p.bloom_slice_min);
    if (p.kway_mode < 0 || p.kway_mode > 2)
        return fail(GR_E_INVALID, "kway_mode %d not in {0, 1, 2}", p.kway_mode);
    if (p.kway_mode == 1)
        for (int l = 0; l < p.sid_length; ++l)
            if (p.kway_k[l] < 1) return fail(GR_E_INVALID, "kway_k[%d] = %d < 1", l, p.kway_k[l]);
    if (p.kway_mode == 2 && (p.kway_kmax < 1 || !(p.kway_target_fill > 0.0f) || p.kway_target_fill > 1.0f))
        return fail(GR_E_INVALID, "dynamic k-way needs kway_kmax >= 1 and kway_target_fill in (0, 1]");
    if (n_sids < 1 || n_sids > (int64_t)1 << 30)
        return fail(GR_E_INVALID, "n_sids %lld not in [1, 2^30]", (long long)n_sids);
    int bpt = 1;
    while ((1 << bpt) < p.vocab_size) ++bpt;
    if (bpt * p.sid_length > 64)
        return fail(GR_E_UNSUPPORTED, "L * ceil(log2 V) = %d exceeds 64", bpt * p.sid_length);

    gr_trie_builder *b = new (std::nothrow) gr_trie_builder;
    if (!b) return fail(GR_E_NOMEM, "out of host memory");
    try {
        b->p = p;
        b->w_bl = p.bloom_bits / 64;
        b->bpt = bpt;
        b->threads = hw_threads(p.n_threads);
        b->n_in = n_sids;
        const int L = p.sid_length;
        std::vector<std::pair<uint64_t, int64_t>> kv((size_t)n_sids);
        for (int64_t i = 0; i < n_sids; ++i) {
            uint64_t key = 0;
            for (int l = 0; l < L; ++l) {
                int32_t tok = sids[i * L + l];
                if (tok < 0 || tok >= p.vocab_size) {
                    delete b;
                    return fail(GR_E_INVALID, "sids[%lld][%d] = %d out of [0, %d)",
                                (long long)i, l, tok, p.vocab_size);
                }
                key = (key << bpt) | (uint64_t)tok;
            }
            kv[i] = {key, i};
        }
        std::sort(kv.begin(), kv.end());
        b->leaf_of_input.assign(n_sids, -1);
        for (int64_t i = 0; i < n_sids; ++i) {
            if (i == 0 || kv[i].first != kv[i - 1].first) b->leaf_key.push_back(kv[i].first);
            b->leaf_of_input[kv[i].second] = (int64_t)b->leaf_key.size() - 1;
        }
        b->n_leaf = (int64_t)b->leaf_key.size();
        // Level sizes and multi-child counts (to reserve room for upper rows).
        b->n_level.assign(L + 1, 0);
        b->n_multi.assign(L + 1, 0);
        b->n_level[0] = 1;
        for (int l = 1; l <= L; ++l) {
            int sh = (L - l) * bpt;
            int64_t n = 0;
            for (int64_t i = 0; i < b->n_leaf; ++i)
                if (i == 0 || (b->leaf_key[i] >> sh) != (b->leaf_key[i - 1] >> sh)) ++n;
            b->n_level[l] = n;
        }
        for (int l = 1; l < L; ++l) {
            // level-l nodes with at least two distinct level-(l+1) children
            int sh1 = (L - l - 1) * bpt;
            int64_t multi = 0, run = 0;
            uint64_t prev_c = 0, prev_p = 0;
            for (int64_t i = 0; i < b->n_leaf; ++i) {
                uint64_t c = b->leaf_key[i] >> sh1;
                if (i > 0 && c == prev_c) continue;
                uint64_t par = c >> bpt;
                if (i > 0 && par == prev_p) {
                    if (++run == 2) ++multi;
                } else {
                    run = 1;
                    prev_p = par;
                }
                prev_c = c;
            }
            b->n_multi[l] = multi;
        }
        int64_t room = b->n_leaf;
        for (int l = 1; l < L; ++l) room += b->n_multi[l];
        b->leaf_bm.assign((size_t)room * p.w_bm, 0);
        if (b->w_bl) b->leaf_bl.assign((size_t)room * b->w_bl, 0);
    } catch (const std::bad_alloc &) {
        delete b;
        return fail(GR_E_NOMEM, "out of host memory building the catalog");
    }
    *out = b;
    return GR_OK;
}

gr_status gr_trie_builder_add_ads(gr_trie_builder *b, int64_t n_ads, const int64_t *ad_sid,
                                  const uint64_t *rules, const int64_t *geo_offsets,
                                  const int32_t *geo_ids) {
    if (!b) return fail(GR_E_INVALID, "gr_trie_builder_add_ads: null builder");
    if (n_ads < 0) return fail(GR_E_INVALID, "n_ads < 0");
    if (n_ads == 0) return GR_OK;
    if (!ad_sid || !rules) return fail(GR_E_INVALID, "gr_trie_builder_add_ads: null array");
    if (b->w_bl && !geo_offsets) return fail(GR_E_INVALID, "geo_offsets is NULL with a Bloom matcher");
    for (int64_t a = 0; a < n_ads; ++a)
        if (ad_sid[a] < 0 || ad_sid[a] >= b->n_in)
            return fail(GR_E_INVALID, "ad_sid[%lld] = %lld out of [0, %lld)", (long long)a,
                        (long long)ad_sid[a], (long long)b->n_in);
    if (b->w_bl) {
        if (geo_offsets[0] < 0) return fail(GR_E_INVALID, "geo_offsets[0] < 0");
        for (int64_t a = 0; a < n_ads; ++a)
            if (geo_offsets[a + 1] < geo_offsets[a])
                return fail(GR_E_INVALID, "geo_offsets decreases at %lld", (long long)a);
        if (geo_offsets[n_ads] > geo_offsets[0] && !geo_ids)
            return fail(GR_E_INVALID, "geo_ids is NULL");
        for (int64_t j = geo_offsets[0]; j < geo_offsets[n_ads]; ++j)
            if (geo_ids[j] < 0) return fail(GR_E_INVALID, "geo_ids[%lld] < 0", (long long)j);
    }
    const int wbm = b->p.w_bm, wbl = b->w_bl, k = b->p.bloom_k;
    const uint32_t wbits = (uint32_t)b->p.bloom_bits;
    uint64_t *lbm = b->leaf_bm.data();
    uint64_t *lbl = b->leaf_bl.data();
    const int64_t *leaf_of = b->leaf_of_input.data();
    parallel_for(n_ads, b->threads, [&](int64_t a0, int64_t a1) {
        uint32_t pos[16];
        for (int64_t a = a0; a < a1; ++a) {
            int64_t leaf = leaf_of[ad_sid[a]];
            for (int w = 0; w < wbm; ++w) {
                uint64_t r = rules[a * wbm + w];
                if (r) __atomic_fetch_or(&lbm[leaf * wbm + w], r, __ATOMIC_RELAXED);
            }
            if (!wbl) continue;
            uint64_t *row = lbl + leaf * wbl;
            for (int64_t j = geo_offsets[a]; j < geo_offsets[a + 1]; ++j) {
                bloom_pos((uint64_t)geo_ids[j], wbits, k, pos);
                for (int i = 0; i < k; ++i) {
                    uint64_t bit = 1ull << (pos[i] & 63);
                    uint64_t *wd = row + (pos[i] >> 6);
                    if (!(__atomic_load_n(wd, __ATOMIC_RELAXED) & bit))
                        __atomic_fetch_or(wd, bit, __ATOMIC_RELAXED);
                }
            }
        }
    });
    return GR_OK;
}

void gr_trie_builder_destroy(gr_trie_builder *b) { delete b; }

static void free_trie_dev(gr_trie *t) {
    if (!t) return;
    hipFree((void *)t->d.node_offsets);
    hipFree((void *)t->d.child_nodes);
    hipFree((void *)t->d.tokens);
    hipFree((void *)t->d.bitmask_index);
    hipFree((void *)t->d.bloom_index);
    hipFree((void *)t->d.bitmask_table);
    hipFree((void *)t->d.bloom_table);
    hipFree((void *)t->d.node_slice);
    hipFree((void *)t->d.slice_table);
    hipFree((void *)t->d.entry_bitmask);
    hipFree((void *)t->d.kway_offsets);
    hipFree((void *)t->d.kway_bmi);
    hipFree((void *)t->d.kway_bli);
    t->d = TrieDev{};
}

// Bit-sliced matcher blocks (a column-major copy of the children's rows).
// A node with c >= min_c child entries gets a block of Wc = ceil(c / 64)
// words per matcher bit position: first bloom_bits positions of the Bloom
// rows (if any), then 64 * w_bm positions of the bitmask rows.  Word
// pos * Wc + (j >> 6) has bit j & 63 set iff bit pos of child entry j's row
// is set.  One block answers eqs 5 and 8 for all of a node's children at
// once: AND the columns of the user's bitmask bits, AND the columns of a
// location's probe positions and OR over locations.  The total is kept
// under MAX_SLICE_WORDS by raising min_c.  A block answers a probe with one
// column of ceil(c / 64) words but moves a whole cache line for it, so it
// pays off over the per-child rows only for wide nodes: 48 children was the
// fastest threshold measured on the main workload (16, 48, 96 and 160 tried).
constexpr int DEFAULT_SLICE_MIN = 48;
constexpr int64_t MAX_SLICE_WORDS = (int64_t)4 << 30;  // 32 GiB

static void build_slices(int64_t num_nodes, const int32_t *off, const int32_t *bmi,
                         const uint64_t *bm, int w_bm, const int32_t *bli, const uint64_t *bl,
                         int w_bl, int bloom_bits, int min_c, int threads,
                         std::vector<int64_t> &node_slice, std::vector<uint64_t> &tab) {
    const int64_t npos = (int64_t)(w_bl ? bloom_bits : 0) + 64 * w_bm;
    node_slice.assign((size_t)num_nodes, -1);
    int64_t total = 0;
    for (;;) {
        total = 0;
        for (int64_t n = 0; n < num_nodes; ++n) {
            const int c = off[n + 1] - off[n];
            if (c >= min_c) total += npos * ((c + 63) / 64);
        }
        if (total <= MAX_SLICE_WORDS) break;
        min_c *= 2;
    }
    total = 0;
    for (int64_t n = 0; n < num_nodes; ++n) {
        const int c = off[n + 1] - off[n];
        if (c >= min_c) {
            node_slice[n] = total;
            total += npos * ((c + 63) / 64);
        }
    }
    tab.assign((size_t)total + 4, 0ull);   // + a tail pad for 4-word column reads
    int64_t *ns = node_slice.data();
    uint64_t *tb = tab.data();
    const int bl_pos = w_bl ? bloom_bits : 0;
    parallel_for(num_nodes, threads, [&](int64_t n0, int64_t n1) {
        auto scatter = [](uint64_t *blk, int64_t wc, int j, const uint64_t *row, int words) {
            const uint64_t bit = 1ull << (j & 63);
            for (int w = 0; w < words; ++w) {
                uint64_t word = row[w];
                while (word) {
                    const int b = __builtin_ctzll(word);
                    blk[(int64_t)(w * 64 + b) * wc + (j >> 6)] |= bit;
                    word &= word - 1;
                }
            }
        };
        for (int64_t n = n0; n < n1; ++n) {
            if (ns[n] < 0) continue;
            const int c = off[n + 1] - off[n];
            const int64_t wc = (c + 63) / 64;
            uint64_t *blk = tb + ns[n];
            for (int j = 0; j < c; ++j) {
                const int32_t e = off[n] + j;
                if (w_bl) scatter(blk, wc, j, bl + (size_t)bli[e] * w_bl, w_bl);
                scatter(blk + (int64_t)bl_pos * wc, wc, j, bm + (size_t)bmi[e] * w_bm, w_bm);
            }
        }
    });
}

// k-way partitioned matchers (GRACE Section 4.2 and Figure 3).  A node's
// descendant SIDs are the sorted leaves below it (a contiguous range); each
// goes, in ascending order, to the partition whose union has the fewest set
// bits after adding it (bitmask and Bloom words together; the lowest index
// on a tie); empty partitions are dropped.  Static: k = kway_k[depth - 1].
// Dynamic: k = 1, 2, 4, ... until the partitions' mean fill is at most the
// target or k reaches kway_kmax.  k never exceeds the node's SID count.  The
// partition unions go to the same deduplicated tables as the other rows.
struct KwayOut {
    std::vector<int32_t> off, bmi, bli;
};

static void kway_partitions(const gr_trie_params &p, int depth, const uint64_t *const *leaf_bm,
                            const uint64_t *const *leaf_bl, int64_t lo, int64_t hi, int wbm,
                            int wbl, std::vector<uint64_t> &out_rows, int &out_n) {
    const int W = wbm + wbl;
    const int64_t n = hi - lo;
    auto greedy = [&](int k, std::vector<uint64_t> &P, std::vector<int64_t> &ones,
                      std::vector<int> &used) {
        P.assign((size_t)k * W, 0ull);
        ones.assign(k, 0);
        used.assign(k, 0);
        for (int64_t i = lo; i < hi; ++i) {
            const uint64_t *bm = leaf_bm[i - lo], *bl = wbl ? leaf_bl[i - lo] : nullptr;
            int best = 0;
            int64_t best_c = INT64_MAX;
            for (int j = 0; j < k; ++j) {
                const uint64_t *r = &P[(size_t)j * W];
                int64_t c = 0;
                for (int w = 0; w < wbm; ++w) c += __builtin_popcountll(r[w] | bm[w]);
                for (int w = 0; w < wbl; ++w) c += __builtin_popcountll(r[wbm + w] | bl[w]);
                if (c < best_c) {
                    best_c = c;
                    best = j;
                }
            }
            uint64_t *r = &P[(size_t)best * W];
            for (int w = 0; w < wbm; ++w) r[w] |= bm[w];
            for (int w = 0; w < wbl; ++w) r[wbm + w] |= bl[w];
            ones[best] = best_c;
            used[best] = 1;
        }
    };
    std::vector<uint64_t> P;
    std::vector<int64_t> ones;
    std::vector<int> used;
    if (p.kway_mode == 1) {
        greedy((int)std::min<int64_t>(p.kway_k[depth - 1], n), P, ones, used);
    } else {
        const int kcap = (int)std::min<int64_t>(p.kway_kmax, n);
        for (int k = 1;; k = std::min(2 * k, kcap)) {
            greedy(k, P, ones, used);
            int64_t tot = 0, nu = 0;
            for (int j = 0; j < k; ++j) {
                tot += ones[j];
                nu += used[j];
            }
            const double fill = (double)tot / ((double)nu * 64.0 * W);
            if (fill <= p.kway_target_fill || k >= kcap) break;
        }
    }
    out_rows.clear();
    out_n = 0;
    for (size_t j = 0; j < used.size(); ++j)
        if (used[j]) {
            out_rows.insert(out_rows.end(), P.begin() + (ptrdiff_t)(j * W), P.begin() + (ptrdiff_t)((j + 1) * W));
            ++out_n;
        }
}

// Appends row r to table T (deduplicated); returns its id.
static int32_t table_add(RowTable &T, const uint64_t *r) {
    if ((size_t)(T.n + 1) * T.w > T.rows.size()) T.rows.resize(((size_t)T.n + 1) * T.w * 2);
    std::memcpy(&T.rows[(size_t)T.n * T.w], r, sizeof(uint64_t) * T.w);
    return T.insert(&T.rows[(size_t)T.n * T.w]);
}

static void build_kway(const gr_trie_params &p, int L, int bpt, int wbm, int wbl,
                       const std::vector<uint64_t> &leaf_key,
                       const std::vector<std::vector<uint64_t>> &pk, const std::vector<int64_t> &base,
                       int64_t num_entries, const std::vector<int32_t> &bmi,
                       const std::vector<int32_t> &bli, std::vector<uint64_t> &bm_store,
                       int64_t &bm_rows, std::vector<uint64_t> &bl_store, int64_t &bl_rows,
                       int threads, KwayOut &o) {
    const int64_t n_leaf = (int64_t)leaf_key.size();
    // the tables as they stand, then the partition unions appended
    auto reopen = [](RowTable &T, std::vector<uint64_t> &store, int w, int64_t n) {
        T.rows.swap(store);
        T.init(w, n * 2);
        for (int64_t r = 0; r < n; ++r) T.insert(&T.rows[(size_t)r * w]);
    };
    RowTable tbm, tbl;
    reopen(tbm, bm_store, wbm, bm_rows);
    if (wbl) reopen(tbl, bl_store, wbl, bl_rows);
    // each leaf's own rows (pointers into the tables, stable while rows only
    // get appended in the serial merge: copied up front)
    std::vector<uint64_t> lbm((size_t)n_leaf * wbm), lbl((size_t)n_leaf * wbl);
    for (int64_t i = 0; i < n_leaf; ++i) {
        const int64_t e = base[L] + i - 1;
        std::memcpy(&lbm[(size_t)i * wbm], &tbm.rows[(size_t)bmi[e] * wbm], sizeof(uint64_t) * wbm);
        if (wbl) std::memcpy(&lbl[(size_t)i * wbl], &tbl.rows[(size_t)bli[e] * wbl], sizeof(uint64_t) * wbl);
    }
    std::vector<const uint64_t *> pbm((size_t)n_leaf), pbl((size_t)n_leaf);
    for (int64_t i = 0; i < n_leaf; ++i) {
        pbm[i] = &lbm[(size_t)i * wbm];
        pbl[i] = wbl ? &lbl[(size_t)i * wbl] : nullptr;
    }
    o.off.assign((size_t)num_entries + 1, 0);
    o.bmi.clear();
    o.bli.clear();
    const int W = wbm + wbl;
    for (int l = 1; l <= L; ++l) {
        const int sh = (L - l) * bpt;
        const int64_t nn = (int64_t)pk[l].size();
        std::vector<int64_t> lo((size_t)nn), hi((size_t)nn);
        for (int64_t i = 0, j = 0; i < nn; ++i) {
            lo[i] = j;
            while (j < n_leaf && (leaf_key[j] >> sh) == pk[l][i]) ++j;
            hi[i] = j;
        }
        const int64_t CH = 4096;   // nodes per parallel batch, merged serially
        std::vector<std::vector<uint64_t>> rows((size_t)CH);
        std::vector<int> cnt((size_t)CH);
        for (int64_t c0 = 0; c0 < nn; c0 += CH) {
            const int64_t c1 = std::min(nn, c0 + CH);
            parallel_for(c1 - c0, threads, [&](int64_t a, int64_t b2) {
                for (int64_t q = a; q < b2; ++q) {
                    const int64_t i = c0 + q;
                    kway_partitions(p, l, pbm.data() + lo[i], pbl.data() + lo[i], lo[i], hi[i], wbm,
                                    wbl, rows[(size_t)q], cnt[(size_t)q]);
                }
            });
            for (int64_t q = 0; q < c1 - c0; ++q) {
                const int64_t e = base[l] + c0 + q - 1;   // entry of node base[l] + i
                for (int j = 0; j < cnt[(size_t)q]; ++j) {
                    const uint64_t *r = &rows[(size_t)q][(size_t)j * W];
                    o.bmi.push_back(table_add(tbm, r));
                    if (wbl) o.bli.push_back(table_add(tbl, r + wbm));
                }
                o.off[(size_t)e + 1] = (int32_t)o.bmi.size();
            }
        }
    }
    for (int64_t e = 1; e <= num_entries; ++e)   // entries are filled in order
        if (o.off[(size_t)e] < o.off[(size_t)e - 1]) o.off[(size_t)e] = o.off[(size_t)e - 1];
    tbm.rows.resize((size_t)tbm.n * wbm);
    bm_store.swap(tbm.rows);
    bm_rows = tbm.n;
    if (wbl) {
        tbl.rows.resize((size_t)tbl.n * wbl);
        bl_store.swap(tbl.rows);
        bl_rows = tbl.n;
    }
}

static gr_status upload_trie(gr_trie *t, const int32_t *off, const int32_t *child,
                             const int16_t *tok, const int32_t *bmi, const int32_t *bli,
                             const uint64_t *bm, const uint64_t *bl, int slice_min,
                             int threads, const int32_t *kw_off = nullptr,
                             const int32_t *kw_bmi = nullptr, const int32_t *kw_bli = nullptr,
                             int64_t kw_rows = 0) {
    hipError_t e;
    int32_t *d_off, *d_child, *d_bmi, *d_bli = nullptr;
    int16_t *d_tok;
    uint64_t *d_bm, *d_bl = nullptr;
    TrieDev &d = t->d;
    hipGetDevice(&t->device);
    if ((e = upload(&d_off, off, (size_t)d.num_nodes + 1)) != hipSuccess) goto err;
    d.node_offsets = d_off;
    if ((e = upload(&d_child, child, (size_t)d.num_entries)) != hipSuccess) goto err;
    d.child_nodes = d_child;
    if ((e = upload(&d_tok, tok, (size_t)d.num_entries)) != hipSuccess) goto err;
    d.tokens = d_tok;
    if ((e = upload(&d_bmi, bmi, (size_t)d.num_entries)) != hipSuccess) goto err;
    d.bitmask_index = d_bmi;
    if ((e = upload(&d_bm, bm, (size_t)d.bm_rows * d.w_bm)) != hipSuccess) goto err;
    d.bitmask_table = d_bm;
    if (d.w_bm <= ENTRY_BM_MAX_W && d.num_entries > 0) {
        std::vector<uint64_t> ebm;
        try {
            ebm.resize((size_t)d.num_entries * d.w_bm);
        } catch (const std::bad_alloc &) {
            free_trie_dev(t);
            return fail(GR_E_NOMEM, "out of host memory building the entry-ordered bitmask rows");
        }
        const int wb = d.w_bm;
        uint64_t *eb = ebm.data();
        parallel_for(d.num_entries, threads, [&](int64_t e0, int64_t e1) {
            for (int64_t j = e0; j < e1; ++j)
                for (int w = 0; w < wb; ++w) eb[j * wb + w] = bm[(size_t)bmi[j] * wb + w];
        });
        uint64_t *d_ebm;
        if ((e = upload(&d_ebm, ebm.data(), ebm.size())) != hipSuccess) goto err;
        d.entry_bitmask = d_ebm;
    }
    if (d.w_bl) {
        if ((e = upload(&d_bli, bli, (size_t)d.num_entries)) != hipSuccess) goto err;
        d.bloom_index = d_bli;
        if ((e = upload(&d_bl, bl, (size_t)d.bl_rows * d.w_bl)) != hipSuccess) goto err;
        d.bloom_table = d_bl;
    }
    if (kw_off) {   // k-way partitions replace the one-union rows in the kernels
        int32_t *d_kwo, *d_kwb, *d_kwl = nullptr;
        if ((e = upload(&d_kwo, kw_off, (size_t)d.num_entries + 1)) != hipSuccess) goto err;
        d.kway_offsets = d_kwo;
        if ((e = upload(&d_kwb, kw_bmi, (size_t)kw_rows)) != hipSuccess) goto err;
        d.kway_bmi = d_kwb;
        if (d.w_bl) {
            if ((e = upload(&d_kwl, kw_bli, (size_t)kw_rows)) != hipSuccess) goto err;
            d.kway_bli = d_kwl;
        }
        d.kway_rows = kw_rows;
        slice_min = -1;   // the bit-sliced blocks hold one-union rows only
    }
    {   // are the root's children nodes 1..n1 (token order)?
        const int32_t n1 = d.num_nodes > 0 ? off[1] - off[0] : 0;
        bool dense = n1 > 0;
        for (int32_t j = 0; j < n1 && dense; ++j) dense = child[off[0] + j] == j + 1;
        d.n_root = dense ? n1 : 0;
    }
    if (slice_min >= 0) {
        std::vector<int64_t> ns;
        std::vector<uint64_t> tab;
        try {
            build_slices(d.num_nodes, off, bmi, bm, d.w_bm, bli, bl, d.w_bl, d.bloom_bits,
                         slice_min ? slice_min : DEFAULT_SLICE_MIN, threads, ns, tab);
        } catch (const std::bad_alloc &) {
            free_trie_dev(t);
            return fail(GR_E_NOMEM, "out of host memory building bit-sliced matcher blocks");
        }
        if (!tab.empty()) {
            int64_t *d_ns;
            uint64_t *d_tab;
            if ((e = upload(&d_ns, ns.data(), ns.size())) != hipSuccess) goto err;
            d.node_slice = d_ns;
            if ((e = upload(&d_tab, tab.data(), tab.size())) != hipSuccess) goto err;
            d.slice_table = d_tab;
            d.slice_words = (int64_t)tab.size();
        }
    }
    return GR_OK;
err:
    free_trie_dev(t);
    if (e == hipErrorOutOfMemory) return fail(GR_E_NOMEM, "device memory exhausted uploading the trie");
    return hip_fail(e, "uploading the trie");
}

gr_status gr_trie_builder_finish(gr_trie_builder *b, gr_trie **out) {
    if (!b || !out) {
        delete b;
        return fail(GR_E_INVALID, "gr_trie_builder_finish: null argument");
    }
    *out = nullptr;
    gr_trie *t = new (std::nothrow) gr_trie;
    if (!t) {
        delete b;
        return fail(GR_E_NOMEM, "out of host memory");
    }
    gr_status st = GR_OK;
    try {
        const int L = b->p.sid_length, bpt = b->bpt, wbm = b->p.w_bm, wbl = b->w_bl;
        const uint64_t tokmask = (1ull << bpt) - 1;
        // Node numbering: root 0, then level 1, 2, ..., L in sorted-prefix order
        // (breadth first; a node's children are contiguous and sorted by token).
        std::vector<int64_t> base(L + 2, 0);
        base[0] = 0;
        base[1] = 1;
        for (int l = 1; l <= L; ++l) base[l + 1] = base[l] + b->n_level[l];
        const int64_t num_nodes = base[L + 1];
        const int64_t num_entries = num_nodes - 1;
        if (num_nodes > INT32_MAX) {
            delete b;
            delete t;
            return fail(GR_E_UNSUPPORTED, "trie with %lld nodes exceeds int32 ids", (long long)num_nodes);
        }
        // Per level: sorted prefix keys and, for each node, its first child.
        std::vector<int32_t> off((size_t)num_nodes + 1, (int32_t)num_entries);
        std::vector<int32_t> child((size_t)num_entries);
        std::vector<int16_t> tok((size_t)num_entries);
        std::vector<int32_t> depth((size_t)num_nodes), parent((size_t)num_nodes);
        std::vector<int16_t> ntok((size_t)num_nodes);
        depth[0] = 0;
        parent[0] = -1;
        ntok[0] = -1;
        std::vector<std::vector<uint64_t>> pk(L + 1);
        for (int l = 1; l <= L; ++l) {
            int sh = (L - l) * bpt;
            pk[l].reserve((size_t)b->n_level[l]);
            for (int64_t i = 0; i < b->n_leaf; ++i) {
                uint64_t k = b->leaf_key[i] >> sh;
                if (pk[l].empty() || pk[l].back() != k) pk[l].push_back(k);
            }
        }
        // children ranges
        {
            // root's children: all level-1 nodes
            off[0] = 0;
            for (int l = 1; l <= L; ++l) {
                int64_t pi = -1;  // parent index within level l-1
                for (int64_t i = 0; i < (int64_t)pk[l].size(); ++i) {
                    int64_t id = base[l] + i;
                    uint64_t pkey = pk[l][i] >> bpt;
                    if (l == 1) {
                        pi = 0;
                    } else {
                        if (pi < 0 || pk[l - 1][pi] != pkey) {
                            ++pi;
                            while (pk[l - 1][pi] != pkey) ++pi;  // keys are sorted
                            off[base[l - 1] + pi] = (int32_t)(id - 1);
                        }
                    }
                    int64_t pid = (l == 1) ? 0 : base[l - 1] + pi;
                    depth[id] = l;
                    parent[id] = (int32_t)pid;
                    ntok[id] = (int16_t)(pk[l][i] & tokmask);
                    child[id - 1] = (int32_t)id;
                    tok[id - 1] = (int16_t)(pk[l][i] & tokmask);
                }
            }
            // nodes with children got their first entry; leaves keep
            // num_entries; make offsets non-decreasing by a backward pass.
            for (int64_t n = num_nodes - 1; n >= 0; --n)
                if (off[n] > off[n + 1]) off[n] = off[n + 1];
        }
        // Matcher rows: leaves from the ads, then each upper node = OR of its
        // children (a single-child node reuses its child's row id).
        auto build_rows = [&](std::vector<uint64_t> &store, int w, std::vector<int32_t> &idx) {
            RowTable tab;
            tab.rows.swap(store);
            tab.init(w, b->n_leaf);
            std::vector<int32_t> rid((size_t)num_nodes, -1);
            for (int64_t i = 0; i < b->n_leaf; ++i)
                rid[base[L] + i] = tab.insert(&tab.rows[(size_t)i * w]);
            std::vector<uint64_t> tmp((size_t)w);
            for (int l = L - 1; l >= 1; --l) {
                for (int64_t i = 0; i < b->n_level[l]; ++i) {
                    int64_t id = base[l] + i;
                    int64_t c0 = off[id] + 1, c1 = off[id + 1] + 1;  // child node ids
                    if (c1 - c0 == 1) {
                        rid[id] = rid[c0];
                        continue;
                    }
                    std::fill(tmp.begin(), tmp.end(), 0ull);
                    for (int64_t c = c0; c < c1; ++c) {
                        const uint64_t *r = &tab.rows[(size_t)rid[c] * w];
                        for (int q = 0; q < w; ++q) tmp[q] |= r[q];
                    }
                    if ((size_t)(tab.n + 1) * w > tab.rows.size()) tab.rows.resize((size_t)(tab.n + 1) * w * 2);
                    std::memcpy(&tab.rows[(size_t)tab.n * w], tmp.data(), sizeof(uint64_t) * w);
                    rid[id] = tab.insert(&tab.rows[(size_t)tab.n * w]);
                }
            }
            idx.resize((size_t)num_entries);
            for (int64_t j = 0; j < num_entries; ++j) idx[j] = rid[j + 1];
            tab.rows.resize((size_t)tab.n * w);
            tab.rows.shrink_to_fit();
            store.swap(tab.rows);
            return tab.n;
        };
        std::vector<int32_t> bmi, bli;
        int64_t bm_rows = build_rows(b->leaf_bm, wbm, bmi);
        int64_t bl_rows = 0;
        if (wbl) bl_rows = build_rows(b->leaf_bl, wbl, bli);
        KwayOut kw;
        if (b->p.kway_mode)
            build_kway(b->p, L, bpt, wbm, wbl, b->leaf_key, pk, base, num_entries, bmi, bli,
                       b->leaf_bm, bm_rows, b->leaf_bl, bl_rows, b->threads, kw);

        TrieDev &d = t->d;
        d.kway_rows = (int64_t)kw.bmi.size();
        d.V = b->p.vocab_size;
        d.L = L;
        d.w_bm = wbm;
        d.w_bl = wbl;
        d.bloom_bits = b->p.bloom_bits;
        d.bloom_k = wbl ? b->p.bloom_k : 0;
        d.num_nodes = num_nodes;
        d.num_entries = num_entries;
        d.bm_rows = bm_rows;
        d.bl_rows = bl_rows;
        t->host_only = b->p.host_only != 0;
        if (!t->host_only)
            st = upload_trie(t, off.data(), child.data(), tok.data(), bmi.data(),
                             wbl ? bli.data() : nullptr, b->leaf_bm.data(),
                             wbl ? b->leaf_bl.data() : nullptr, b->p.bloom_slice_min, b->threads,
                             b->p.kway_mode ? kw.off.data() : nullptr, kw.bmi.data(),
                             wbl ? kw.bli.data() : nullptr, (int64_t)kw.bmi.size());
        if (st == GR_OK && (b->p.keep_host || t->host_only)) {
            t->has_host = true;
            t->h_off.swap(off);
            t->h_child.swap(child);
            t->h_tok.swap(tok);
            t->h_bmi.swap(bmi);
            t->h_bli.swap(bli);
            t->h_bm.swap(b->leaf_bm);
            t->h_bl.swap(b->leaf_bl);
            t->h_depth.swap(depth);
            t->h_parent.swap(parent);
            t->h_ntok.swap(ntok);
            t->h_kw_off.swap(kw.off);
            t->h_kw_bmi.swap(kw.bmi);
            t->h_kw_bli.swap(kw.bli);
        }
    } catch (const std::bad_alloc &) {
        st = fail(GR_E_NOMEM, "out of host memory finishing the trie");
    }
    delete b;
    if (st != GR_OK) {
        free_trie_dev(t);
        delete t;
        return st;
    }
    *out = t;
    return GR_OK;
}

gr_status gr_trie_create(const gr_trie_view *a, gr_trie **out) {
    if (!a || !out) return fail(GR_E_INVALID, "gr_trie_create: null argument");
    *out = nullptr;
    if (a->vocab_size < 2 || a->vocab_size > 32768) return fail(GR_E_INVALID, "vocab_size %d not in [2, 32768]", a->vocab_size);
    if (a->sid_length < 1 || a->sid_length > 16) return fail(GR_E_INVALID, "sid_length %d not in [1, 16]", a->sid_length);
    if (a->w_bm < 1 || a->w_bm > MAX_WBM) return fail(GR_E_INVALID, "w_bm %d not in [1, %d]", a->w_bm, MAX_WBM);
    if (a->bloom_bits && (a->bloom_bits < 64 || a->bloom_bits > 65536 || (a->bloom_bits & (a->bloom_bits - 1))))
        return fail(GR_E_INVALID, "bloom_bits %d is not 0 or a power of two in [64, 65536]", a->bloom_bits);
    if (a->bloom_bits && (a->bloom_k < 1 || a->bloom_k > 16)) return fail(GR_E_INVALID, "bloom_k %d not in [1, 16]", a->bloom_k);
    if (a->num_nodes < 1 || a->num_nodes > INT32_MAX) return fail(GR_E_INVALID, "num_nodes %lld out of range", (long long)a->num_nodes);
    if (a->num_entries < 0 || a->num_entries > INT32_MAX) return fail(GR_E_INVALID, "num_entries %lld out of range", (long long)a->num_entries);
    if (!a->node_offsets || (a->num_entries && (!a->child_nodes || !a->tokens || !a->bitmask_index)))
        return fail(GR_E_INVALID, "gr_trie_create: null array");
    if (a->bm_rows < 1 || !a->bitmask_table) return fail(GR_E_INVALID, "bitmask table is empty");
    const bool bloom = a->bloom_bits != 0;
    if (bloom && (a->bl_rows < 1 || !a->bloom_table || (a->num_entries && !a->bloom_index)))
        return fail(GR_E_INVALID, "bloom table or index missing");
    if (a->node_offsets[0] != 0) return fail(GR_E_INVALID, "node_offsets[0] = %d, expected 0", a->node_offsets[0]);
    if (a->node_offsets[a->num_nodes] != a->num_entries)
        return fail(GR_E_INVALID, "node_offsets[num_nodes] = %d, expected num_entries", a->node_offsets[a->num_nodes]);
    for (int64_t n = 0; n < a->num_nodes; ++n) {
        int32_t s = a->node_offsets[n], e = a->node_offsets[n + 1];
        if (e < s) return fail(GR_E_INVALID, "node_offsets decreases at node %lld", (long long)n);
        for (int32_t j = s; j < e; ++j) {
            if (a->child_nodes[j] < 1 || a->child_nodes[j] >= a->num_nodes)
                return fail(GR_E_INVALID, "child_nodes[%d] = %d out of [1, %lld)", j, a->child_nodes[j], (long long)a->num_nodes);
            if (a->tokens[j] < 0 || a->tokens[j] >= a->vocab_size)
                return fail(GR_E_INVALID, "tokens[%d] = %d out of [0, %d)", j, a->tokens[j], a->vocab_size);
            if (j > s && a->tokens[j] <= a->tokens[j - 1])
                return fail(GR_E_INVALID, "tokens of node %lld not strictly increasing at entry %d", (long long)n, j);
            if (a->bitmask_index[j] < 0 || a->bitmask_index[j] >= a->bm_rows)
                return fail(GR_E_INVALID, "bitmask_index[%d] = %d out of range", j, a->bitmask_index[j]);
            if (bloom && (a->bloom_index[j] < 0 || a->bloom_index[j] >= a->bl_rows))
                return fail(GR_E_INVALID, "bloom_index[%d] = %d out of range", j, a->bloom_index[j]);
        }
    }
    if (a->kway_offsets) {   // optional k-way partitions
        if (a->kway_offsets[0] != 0 || a->kway_offsets[a->num_entries] != a->kway_rows ||
            a->kway_rows < 0 || !a->kway_bitmask_index || (bloom && !a->kway_bloom_index))
            return fail(GR_E_INVALID, "k-way offsets do not span [0, kway_rows) or an index is missing");
        for (int64_t e = 0; e < a->num_entries; ++e)
            if (a->kway_offsets[e + 1] < a->kway_offsets[e])
                return fail(GR_E_INVALID, "kway_offsets decreases at entry %lld", (long long)e);
        for (int64_t q = 0; q < a->kway_rows; ++q)
            if (a->kway_bitmask_index[q] < 0 || a->kway_bitmask_index[q] >= a->bm_rows ||
                (bloom && (a->kway_bloom_index[q] < 0 || a->kway_bloom_index[q] >= a->bl_rows)))
                return fail(GR_E_INVALID, "k-way matcher id %lld out of range", (long long)q);
    }
    gr_trie *t = new (std::nothrow) gr_trie;
    if (!t) return fail(GR_E_NOMEM, "out of host memory");
    TrieDev &d = t->d;
    d.V = a->vocab_size;
    d.L = a->sid_length;
    d.w_bm = a->w_bm;
    d.w_bl = a->bloom_bits / 64;
    d.bloom_bits = a->bloom_bits;
    d.bloom_k = bloom ? a->bloom_k : 0;
    d.num_nodes = a->num_nodes;
    d.num_entries = a->num_entries;
    d.bm_rows = a->bm_rows;
    d.bl_rows = bloom ? a->bl_rows : 0;
    gr_status st = upload_trie(t, a->node_offsets, a->child_nodes, a->tokens, a->bitmask_index,
                               a->bloom_index, a->bitmask_table, a->bloom_table, 0, hw_threads(0),
                               a->kway_offsets, a->kway_bitmask_index,
                               bloom ? a->kway_bloom_index : nullptr, a->kway_rows);
    if (st != GR_OK) {
        delete t;
        return st;
    }
    *out = t;
    return GR_OK;
}

static void fill_sizes(const gr_trie *t, gr_trie_view *o) {
    std::memset(o, 0, sizeof *o);
    o->vocab_size = t->d.V;
    o->sid_length = t->d.L;
    o->w_bm = t->d.w_bm;
    o->bloom_bits = t->d.bloom_bits;
    o->bloom_k = t->d.bloom_k;
    o->num_nodes = t->d.num_nodes;
    o->num_entries = t->d.num_entries;
    o->bm_rows = t->d.bm_rows;
    o->bl_rows = t->d.bl_rows;
    o->slice_words = t->d.slice_words;
    o->kway_rows = t->d.kway_rows;
}

gr_status gr_trie_info(const gr_trie *t, gr_trie_view *o) {
    if (!t || !o) return fail(GR_E_INVALID, "gr_trie_info: null argument");
    fill_sizes(t, o);
    return GR_OK;
}

gr_status gr_trie_host_view(const gr_trie *t, gr_trie_view *o) {
    if (!t || !o) return fail(GR_E_INVALID, "gr_trie_host_view: null argument");
    if (!t->has_host) return fail(GR_E_INVALID, "trie was built without keep_host");
    fill_sizes(t, o);
    o->node_offsets = t->h_off.data();
    o->child_nodes = t->h_child.data();
    o->tokens = t->h_tok.data();
    o->bitmask_index = t->h_bmi.data();
    o->bloom_index = t->h_bli.empty() ? nullptr : t->h_bli.data();
    o->bitmask_table = t->h_bm.data();
    o->bloom_table = t->h_bl.empty() ? nullptr : t->h_bl.data();
    o->node_depth = t->h_depth.data();
    o->node_parent = t->h_parent.data();
    o->node_token = t->h_ntok.data();
    o->kway_offsets = t->h_kw_off.empty() ? nullptr : t->h_kw_off.data();
    o->kway_bitmask_index = t->h_kw_bmi.empty() ? nullptr : t->h_kw_bmi.data();
    o->kway_bloom_index = t->h_kw_bli.empty() ? nullptr : t->h_kw_bli.data();
    return GR_OK;
}

void gr_trie_destroy(gr_trie *t) {
    if (!t) return;
    free_trie_dev(t);
    delete t;
}

// ---------------------------------------------------------------------------
// Hot path entry points
// ---------------------------------------------------------------------------

static bool dtype_ok(gr_dtype d) { return d == GR_F32 || d == GR_BF16; }

// Shapes the self-attention kernels take: a head is d_h / vec pieces of
// vec elements (4 bf16 or 2 fp32) spread over a power-of-two group of lanes,
// whose dot products are summed by a butterfly over that group, and a row
// of H * d_h elements fits 16 pieces on each of the 64 lanes.
static gr_status check_self_shape(const char *fn, int H, int d, gr_dtype dt) {
    const int vec = dt == GR_BF16 ? 4 : 2;
    if (d % vec || d / vec > 64 || (d / vec & (d / vec - 1)))
        return fail(GR_E_UNSUPPORTED, "%s: self-attention d_h %d unsupported for this dtype "
                    "(a multiple of %d with d_h / %d a power of two <= 64)", fn, d, vec, vec);
    if ((int64_t)H * d > 64 * vec * 16)
        return fail(GR_E_UNSUPPORTED, "%s: H*d_h %lld too large for self-attention", fn,
                    (long long)H * d);
    return GR_OK;
}

// The bf16 cross-attention tiles read one request's queries and one
// (request, head)'s context through buffer descriptors whose extent is a
// 32-bit byte count: M*H*d_h and T_ctx*d_h bf16 values must stay below 2^32
// bytes.
static gr_status check_cross_extent(const char *fn, int M, int H, int T, int d, gr_dtype dt) {
    if (dt != GR_BF16) return GR_OK;
    const int64_t lim = (int64_t)1 << 32;
    if ((int64_t)M * H * d * 2 >= lim)
        return fail(GR_E_UNSUPPORTED, "%s: one request's queries (M*H*d_h = %lld bf16) exceed 2^32 bytes",
                    fn, (long long)M * H * d);
    if ((int64_t)T * d * 2 >= lim)
        return fail(GR_E_UNSUPPORTED, "%s: one head's context (T_ctx*d_h = %lld bf16) exceeds 2^32 bytes",
                    fn, (long long)T * d);
    return GR_OK;
}

static gr_status check_attn_common(const char *fn, int B, int M, int H, int d, gr_dtype dt) {
    if (!dtype_ok(dt)) return fail(GR_E_INVALID, "%s: unknown dtype %d", fn, (int)dt);
    if (B < 1 || M < 1 || H < 1 || d < 1) return fail(GR_E_INVALID, "%s: non-positive shape", fn);
    return GR_OK;
}

gr_status gr_cross_attn(const void *q, const void *k_ctx, const void *v_ctx, void *out,
                        int32_t B, int32_t M, int32_t H, int32_t T_ctx, int32_t d_h,
                        gr_dtype dtype, void *stream) {
    gr_status st = check_attn_common("gr_cross_attn", B, M, H, d_h, dtype);
    if (st) return st;
    if (!q || !k_ctx || !v_ctx || !out) return fail(GR_E_INVALID, "gr_cross_attn: null pointer");
    if (T_ctx < 1) return fail(GR_E_INVALID, "gr_cross_attn: T_ctx %d < 1", T_ctx);
    if ((int64_t)B * M * H > INT32_MAX) return fail(GR_E_INVALID, "gr_cross_attn: too many rows");
    if (dtype == GR_BF16 && d_h != 32 && d_h != 64 && d_h != 128)
        return fail(GR_E_UNSUPPORTED, "gr_cross_attn: bf16 d_h %d not in {32, 64, 128}", d_h);
    if (dtype == GR_F32 && d_h > 64)
        return fail(GR_E_UNSUPPORTED, "gr_cross_attn: f32 d_h %d > 64", d_h);
    st = check_cross_extent("gr_cross_attn", M, H, T_ctx, d_h, dtype);
    if (st) return st;
    hipError_t e = launch_cross_attn(q, k_ctx, v_ctx, out, B, M, H, T_ctx, d_h, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_cross_attn launch");
    return GR_OK;
}

size_t gr_cross_attn_workspace(int32_t B, int32_t M, int32_t H, int32_t T_ctx, int32_t d_h,
                               gr_dtype dtype) {
    if (B < 1 || M < 1 || H < 1 || T_ctx < 1 || d_h < 1) return 0;
    return cross_split_plan(B, M, H, T_ctx, d_h, dtype).bytes;
}

gr_status gr_cross_attn_ws(const void *q, const void *k_ctx, const void *v_ctx, void *out,
                           int32_t B, int32_t M, int32_t H, int32_t T_ctx, int32_t d_h,
                           gr_dtype dtype, void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return gr_cross_attn(q, k_ctx, v_ctx, out, B, M, H, T_ctx, d_h, dtype, stream);
    gr_status st = check_attn_common("gr_cross_attn_ws", B, M, H, d_h, dtype);
    if (st) return st;
    if (T_ctx < 1) return fail(GR_E_INVALID, "gr_cross_attn_ws: T_ctx %d < 1", T_ctx);
    const CrossSplit pl = cross_split_plan(B, M, H, T_ctx, d_h, dtype);
    if (pl.S < 2) return gr_cross_attn(q, k_ctx, v_ctx, out, B, M, H, T_ctx, d_h, dtype, stream);
    if (!q || !k_ctx || !v_ctx || !out) return fail(GR_E_INVALID, "gr_cross_attn_ws: null pointer");
    if ((int64_t)B * M * H > INT32_MAX) return fail(GR_E_INVALID, "gr_cross_attn_ws: too many rows");
    st = check_cross_extent("gr_cross_attn_ws", M, H, T_ctx, d_h, dtype);
    if (st) return st;
    if (ws_bytes < pl.bytes || ((uintptr_t)ws & 15))
        return fail(GR_E_WORKSPACE, "gr_cross_attn_ws: workspace of %zu bytes (16-byte aligned) needed",
                    pl.bytes);
    hipError_t e = launch_cross_split(q, k_ctx, v_ctx, out, B, M, H, T_ctx, d_h, pl, ws,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_cross_attn_ws launch");
    return GR_OK;
}

gr_status gr_self_attn_paged(const void *q, const void *k_new, const void *v_new,
                             void *k_pool, void *v_pool, int64_t pool_blocks,
                             int32_t *table, int64_t fresh_base, int32_t R, int32_t t,
                             int32_t L, int32_t H, int32_t d_h, gr_dtype dtype,
                             void *out, void *stream) {
    gr_status st = check_attn_common("gr_self_attn_paged", 1, R, H, d_h, dtype);
    if (st) return st;
    if (!q || !k_new || !v_new || !k_pool || !v_pool || !table || !out)
        return fail(GR_E_INVALID, "gr_self_attn_paged: null pointer");
    if (L < 1 || L > 16 || t < 0 || t >= L) return fail(GR_E_INVALID, "gr_self_attn_paged: t %d / L %d invalid", t, L);
    if (fresh_base < 0 || pool_blocks < 0 || fresh_base + R > pool_blocks || fresh_base + R > INT32_MAX)
        return fail(GR_E_INVALID, "gr_self_attn_paged: blocks [%lld, %lld) exceed pool of %lld",
                    (long long)fresh_base, (long long)(fresh_base + R), (long long)pool_blocks);
    st = check_self_shape("gr_self_attn_paged", H, d_h, dtype);
    if (st) return st;
    hipError_t e = launch_self_attn(q, k_new, v_new, k_pool, v_pool, pool_blocks, table, fresh_base, R, t, L, H, d_h,
                                    dtype, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_self_attn_paged launch");
    return GR_OK;
}

gr_status gr_joint_attn(const void *q, const void *k_ctx, const void *v_ctx, const void *k_new,
                        const void *v_new, void *k_pool, void *v_pool, int64_t pool_blocks,
                        int32_t *table, int64_t fresh_base, int32_t B, int32_t M, int32_t H,
                        int32_t T_ctx, int32_t d_h, int32_t t, int32_t L, gr_dtype dtype,
                        void *out, void *stream) {
    gr_status st = check_attn_common("gr_joint_attn", B, M, H, d_h, dtype);
    if (st) return st;
    if (!q || !k_ctx || !v_ctx || !k_new || !v_new || !k_pool || !v_pool || !table || !out)
        return fail(GR_E_INVALID, "gr_joint_attn: null pointer");
    if (T_ctx < 1) return fail(GR_E_INVALID, "gr_joint_attn: T_ctx %d < 1", T_ctx);
    if ((int64_t)B * M * H > INT32_MAX) return fail(GR_E_INVALID, "gr_joint_attn: too many rows");
    if (L < 1 || L > 16 || t < 0 || t >= L) return fail(GR_E_INVALID, "gr_joint_attn: t %d / L %d invalid", t, L);
    const int64_t R = (int64_t)B * M;
    if (fresh_base < 0 || pool_blocks < 0 || fresh_base + R > pool_blocks || fresh_base + R > INT32_MAX)
        return fail(GR_E_INVALID, "gr_joint_attn: blocks [%lld, %lld) exceed pool of %lld",
                    (long long)fresh_base, (long long)(fresh_base + R), (long long)pool_blocks);
    if (dtype == GR_BF16 && d_h != 32 && d_h != 64 && d_h != 128)
        return fail(GR_E_UNSUPPORTED, "gr_joint_attn: bf16 d_h %d not in {32, 64, 128}", d_h);
    if (dtype == GR_F32 && d_h > 64)
        return fail(GR_E_UNSUPPORTED, "gr_joint_attn: f32 d_h %d > 64", d_h);
    st = check_cross_extent("gr_joint_attn", M, H, T_ctx, d_h, dtype);
    if (st) return st;
    hipError_t e = launch_joint_attn(q, k_ctx, v_ctx, k_new, v_new, k_pool, v_pool, pool_blocks, table,
                                     fresh_base, B, M, H, T_ctx, d_h, t, L, dtype, out,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_joint_attn launch");
    return GR_OK;
}

}  // extern "C"

namespace gr {
TailWsLayout tail_ws_layout(int32_t B, int32_t M_in, int32_t V) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    TailWsLayout l{};
    l.shape = tail_shape(B, M_in, V);
    const size_t nseg = (size_t)B * l.shape.gx;
    const size_t nsurv = nseg * (size_t)l.shape.seg_cap;
    size_t o = 0;
    // the histograms, the segments' back counts and the cutoff counters
    // first, at fixed places and sizes: each region is only ever used as what
    // it is and stays zero between calls of any shape; then the inverse map of root children at a
    // fixed place, so that a decode's steps (several M_in) find it where the
    // previous step left it (its content is checked before use)
    l.hist = o;    o = al(o + sizeof(uint32_t) * (size_t)NBINS * MAX_B);
    l.segback = o; o = al(o + sizeof(uint32_t) * (size_t)MAX_B * NM_MAX_GX);
    l.cut = o;     o = al(o + sizeof(uint32_t) * (size_t)MAX_B * NCUT);
    l.inv = o;     o = al(o + sizeof(int32_t) * (size_t)B * V);
    l.segcnt = o;  o = al(o + sizeof(uint32_t) * nseg);
    l.skey = o;   o = al(o + sizeof(uint64_t) * nsurv);
    l.schild = o; o = al(o + sizeof(int32_t) * nsurv);
    l.sbin = o;   o = al(o + sizeof(uint16_t) * nsurv);
    l.total = o;
    return l;
}
}  // namespace gr

extern "C" {

size_t gr_constrain_topk_workspace(int32_t B, int32_t M_in, int32_t V, int32_t k_out) {
    (void)k_out;
    if (B < 1 || M_in < 1 || V < 1) return 0;
    return tail_ws_layout(B, M_in, V).total;
}

gr_status gr_constrain_topk_shape(int32_t B, int32_t M_in, int32_t V, int32_t *rows_wg,
                                  int32_t *gx, int64_t *seg_cap) {
    if (B < 1 || M_in < 1 || V < 1 || !rows_wg || !gx || !seg_cap)
        return fail(GR_E_INVALID, "gr_constrain_topk_shape: non-positive size or NULL output");
    const TailShape sh = tail_shape(B, M_in, V);
    *rows_wg = sh.rows_wg;
    *gx = sh.gx;
    *seg_cap = sh.seg_cap;
    return GR_OK;
}

static gr_status check_tail(const gr_trie *trie, const gr_tail_args *a, const char *fn,
                            bool caller_ws = true) {
    if (!trie || !a) return fail(GR_E_INVALID, "%s: null argument", fn);
    if (trie->host_only) return fail(GR_E_INVALID, "%s: trie was built host_only", fn);
    const TrieDev &d = trie->d;
    if (!dtype_ok(a->dtype)) return fail(GR_E_INVALID, "%s: unknown dtype %d", fn, (int)a->dtype);
    if (a->B < 1 || a->M_in < 1 || a->k_out < 1) return fail(GR_E_INVALID, "%s: B, M_in, k_out must be >= 1", fn);
    if (a->B > MAX_B) return fail(GR_E_UNSUPPORTED, "%s: B %d > %d", fn, a->B, MAX_B);
    if (a->V != d.V) return fail(GR_E_INVALID, "%s: V %d differs from the trie's %d", fn, a->V, d.V);
    if (a->V > MAX_V) return fail(GR_E_UNSUPPORTED, "%s: V %d > %d", fn, a->V, MAX_V);
    if (a->k_out > MAX_K) return fail(GR_E_UNSUPPORTED, "%s: k_out %d > %d", fn, a->k_out, MAX_K);
    if (a->L != d.L || a->t < 0 || a->t >= a->L) return fail(GR_E_INVALID, "%s: t %d / L %d invalid for the trie", fn, a->t, a->L);
    if ((int64_t)a->M_in * a->V > INT32_MAX) return fail(GR_E_UNSUPPORTED, "%s: M_in * V exceeds 2^31", fn);
    if (a->M_in > MAX_M_IN) return fail(GR_E_UNSUPPORTED, "%s: M_in %d > %d", fn, a->M_in, MAX_M_IN);
    if ((int64_t)a->B * a->M_in > INT32_MAX || (int64_t)a->B * a->k_out > INT32_MAX)
        return fail(GR_E_INVALID, "%s: too many rows", fn);
    if (!a->user_bm || !a->logits || !a->node_in || !a->acc_in || !a->parent_out || !a->token_out ||
        !a->node_out || !a->acc_out)
        return fail(GR_E_INVALID, "%s: null pointer", fn);
    if (d.bloom_bits > 32768)
        return fail(GR_E_UNSUPPORTED, "%s: Bloom filters of %d bits exceed the 32768 the tail stages in LDS", fn, d.bloom_bits);
    if (d.w_bl) {
        if (a->n_loc < 0 || (int64_t)a->n_loc * ((d.bloom_k + 3) & ~3) > MAX_PROBES)
            return fail(GR_E_UNSUPPORTED, "%s: n_loc %d * bloom_k %d (rounded up to a multiple of 4) exceeds %d",
                        fn, a->n_loc, d.bloom_k, MAX_PROBES);
        if (a->n_loc > 0 && !a->user_probes) return fail(GR_E_INVALID, "%s: user_probes is NULL", fn);
    }
    if (a->tokens_out && a->t > 0 && !a->tokens_in) return fail(GR_E_INVALID, "%s: tokens_in is NULL", fn);
    if (a->table_out && !a->table_in) return fail(GR_E_INVALID, "%s: table_in is NULL", fn);
    if (!caller_ws) return GR_OK;
    size_t need = tail_ws_layout(a->B, a->M_in, a->V).total;
    if (!a->ws || a->ws_bytes < need)
        return fail(GR_E_WORKSPACE, "%s: workspace %zu bytes < %zu required", fn, a->ws_bytes, need);
    if (((uintptr_t)a->ws & 255) != 0) return fail(GR_E_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
    return GR_OK;
}

gr_status gr_constrain(const gr_trie *trie, const gr_tail_args *a, void *stream) {
    gr_status st = check_tail(trie, a, "gr_constrain");
    if (st) return st;
    hipError_t e = launch_constrain(trie->d, *a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_constrain launch");
    return GR_OK;
}

gr_status gr_topk_reorder(const gr_trie *trie, const gr_tail_args *a, void *stream) {
    gr_status st = check_tail(trie, a, "gr_topk_reorder");
    if (st) return st;
    hipError_t e = launch_topk_reorder(trie->d, *a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_topk_reorder launch");
    return GR_OK;
}

gr_status gr_constrain_topk(const gr_trie *trie, const gr_tail_args *a, void *stream) {
    gr_status st = check_tail(trie, a, "gr_constrain_topk");
    if (st) return st;
    hipError_t e = launch_tail(trie->d, *a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_constrain_topk launch");
    return GR_OK;
}

gr_status gr_constrain_topk_noalloc(const gr_trie *trie, const gr_tail_args *a, void *stream) {
    const char *fn = "gr_constrain_topk_noalloc";
    if (!trie || !a) return fail(GR_E_INVALID, "%s: null argument", fn);
    if (a->B >= 1 && a->M_in >= 1 && a->V >= 1) {
        const size_t need = tail_ws_layout(a->B, a->M_in, a->V).total;
        if (need > TAIL_SCRATCH_BYTES)
            return fail(GR_E_UNSUPPORTED,
                        "%s: B %d x M_in %d x V %d needs %zu bytes of tail scratch, more than the "
                        "%zu the library holds per device (use gr_constrain_topk with a workspace)",
                        fn, a->B, a->M_in, a->V, need, TAIL_SCRATCH_BYTES);
    }
    gr_status st = check_tail(trie, a, fn, false);
    if (st) return st;
    void *ws = nullptr;
    hipError_t e = tail_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "gr_constrain_topk_noalloc: scratch lookup");
    gr_tail_args b = *a;
    b.ws = ws;
    b.ws_bytes = TAIL_SCRATCH_BYTES;
    hipStream_t hs = (hipStream_t)stream;
    // the scratch keeps the last call's contents: clear the histograms this
    // call accumulates into (the rest is written before it is read)
    e = launch_clear_hist(ws, b.B, hs);
    if (e == hipSuccess) e = launch_tail(trie->d, b, hs);
    if (e != hipSuccess) return hip_fail(e, "gr_constrain_topk_noalloc launch");
    return GR_OK;
}

// Validation of one decode step; nothing is launched.
static gr_status check_step(const gr_trie *trie, const gr_step_args *s) {
    if (!trie || !s) return fail(GR_E_INVALID, "gr_decode_step: null argument");
    const gr_tail_args &a = s->tail;
    // The attention shapes first (they need nothing from the trie), then the
    // tail; everything is validated before the first launch.
    gr_status st = check_attn_common("gr_decode_step", a.B, a.M_in, s->H, s->d_h, a.dtype);
    if (st) return st;
    if (!s->k_ctx || !s->v_ctx || !s->qx || !s->q || !s->k_new || !s->v_new || !s->k_pool ||
        !s->v_pool || !s->cross_out || !s->self_out)
        return fail(GR_E_INVALID, "gr_decode_step: null pointer");
    if ((int64_t)a.B * a.M_in > INT32_MAX) return fail(GR_E_INVALID, "gr_decode_step: too many rows");
    const int64_t R = (int64_t)a.B * a.M_in;
    if (s->T_ctx < 1) return fail(GR_E_INVALID, "gr_decode_step: T_ctx < 1");
    if (a.dtype == GR_BF16 && s->d_h != 32 && s->d_h != 64 && s->d_h != 128)
        return fail(GR_E_UNSUPPORTED, "gr_decode_step: bf16 d_h %d not in {32, 64, 128}", s->d_h);
    if (a.dtype == GR_F32 && s->d_h > 64) return fail(GR_E_UNSUPPORTED, "gr_decode_step: f32 d_h > 64");
    st = check_cross_extent("gr_decode_step", a.M_in, s->H, s->T_ctx, s->d_h, a.dtype);
    if (st) return st;
    st = check_self_shape("gr_decode_step", s->H, s->d_h, a.dtype);
    if (st) return st;
    if (s->fresh_base < 0 || s->fresh_base + R > s->pool_blocks || s->fresh_base + R > INT32_MAX)
        return fail(GR_E_INVALID, "gr_decode_step: pool of %lld blocks too small", (long long)s->pool_blocks);
    if (!a.table_in) return fail(GR_E_INVALID, "gr_decode_step: tail.table_in is NULL");
    if (s->attn_ws) {
        const CrossSplit pl = cross_split_plan(a.B, a.M_in, s->H, s->T_ctx, s->d_h, a.dtype);
        if (pl.S > 1 && (s->attn_ws_bytes < pl.bytes || ((uintptr_t)s->attn_ws & 15)))
            return fail(GR_E_WORKSPACE, "gr_decode_step: attention workspace of %zu bytes needed",
                        pl.bytes);
    }
    return check_tail(trie, &a, "gr_decode_step");
}

static gr_status launch_step(const gr_trie *trie, const gr_step_args *s, void *stream) {
    const gr_tail_args &a = s->tail;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    const CrossSplit pl = s->attn_ws
                              ? cross_split_plan(a.B, a.M_in, s->H, s->T_ctx, s->d_h, a.dtype)
                              : CrossSplit{1, s->T_ctx, 0};
    if (pl.S > 1) {
        // few tiles over a long context: the split cross-attention (and its
        // merge), then the self-attention
        e = launch_cross_split(s->qx, s->k_ctx, s->v_ctx, s->cross_out, a.B, a.M_in, s->H,
                               s->T_ctx, s->d_h, pl, s->attn_ws, hs);
        if (e == hipSuccess)
            e = launch_self_attn(s->q, s->k_new, s->v_new, s->k_pool, s->v_pool, s->pool_blocks,
                                 const_cast<int32_t *>(a.table_in), s->fresh_base, a.B * a.M_in,
                                 a.t, a.L, s->H, s->d_h, a.dtype, s->self_out, hs);
        if (e != hipSuccess) return hip_fail(e, "gr_decode_step attention launch");
    } else {
        // A1 and A2 are independent: one launch runs both
        e = launch_attn_pair(s->qx, s->k_ctx, s->v_ctx, s->cross_out, a.B, a.M_in, s->H, s->T_ctx,
                             s->d_h, s->q, s->k_new, s->v_new, s->k_pool, s->v_pool,
                             s->pool_blocks, const_cast<int32_t *>(a.table_in), s->fresh_base,
                             a.t, a.L, a.dtype, s->self_out, hs);
        if (e != hipSuccess) return hip_fail(e, "gr_decode_step attention launch");
    }
    e = launch_tail(trie->d, a, hs);
    if (e != hipSuccess) return hip_fail(e, "gr_decode_step constrain/top-k launch");
    return GR_OK;
}


gr_status gr_decode_step(const gr_trie *trie, const gr_step_args *s, void *stream) {
    gr_status st = check_step(trie, s);
    if (st) return st;
    return launch_step(trie, s, stream);
}

struct gr_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int device = 0;
};

gr_status gr_decode_graph_create(const gr_trie *trie, const gr_step_args *steps, int32_t n_steps,
                                 void *stream, gr_graph **out) {
    if (!out) return fail(GR_E_INVALID, "gr_decode_graph_create: out is NULL");
    *out = nullptr;
    if (!trie || !steps || n_steps < 1) return fail(GR_E_INVALID, "gr_decode_graph_create: no steps");
    if (!stream) return fail(GR_E_INVALID, "gr_decode_graph_create: capture needs a created stream");
    for (int32_t t = 0; t < n_steps; ++t) {
        gr_status st = check_step(trie, &steps[t]);
        if (st) return st;
    }
    hipStream_t hs = (hipStream_t)stream;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(hs, &cs);
    if (e != hipSuccess) return hip_fail(e, "gr_decode_graph_create: stream query");
    if (cs != hipStreamCaptureStatusNone) return fail(GR_E_INVALID, "gr_decode_graph_create: stream is already capturing");
    e = hipStreamBeginCapture(hs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "gr_decode_graph_create: begin capture");
    gr_status st = GR_OK;
    for (int32_t t = 0; t < n_steps && st == GR_OK; ++t) st = launch_step(trie, &steps[t], stream);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(hs, &g);
    if (st != GR_OK || e != hipSuccess) {
        if (g) hipGraphDestroy(g);
        return st != GR_OK ? st : hip_fail(e, "gr_decode_graph_create: end capture");
    }
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        hipGraphDestroy(g);
        return hip_fail(e, "gr_decode_graph_create: instantiate");
    }
    gr_graph *gg = new (std::nothrow) gr_graph;
    if (!gg) {
        hipGraphExecDestroy(x);
        hipGraphDestroy(g);
        return fail(GR_E_NOMEM, "gr_decode_graph_create: out of host memory");
    }
    gg->graph = g;
    gg->exec = x;
    hipGetDevice(&gg->device);
    *out = gg;
    return GR_OK;
}

gr_status gr_decode_graph_launch(const gr_graph *graph, void *stream) {
    if (!graph || !graph->exec) return fail(GR_E_INVALID, "gr_decode_graph_launch: null graph");
    hipError_t e = hipGraphLaunch(graph->exec, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gr_decode_graph_launch");
    return GR_OK;
}

void gr_decode_graph_destroy(gr_graph *graph) {
    if (!graph) return;
    if (graph->exec) hipGraphExecDestroy(graph->exec);
    if (graph->graph) hipGraphDestroy(graph->graph);
    delete graph;
}

}  // extern "C"
