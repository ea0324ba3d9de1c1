// Post stage after decoding (GRACE Section 2.1 steps 3-4, Section 2.2): the
// SID-to-ad index expands each finished SID into its ads and the ads
// targeting index runs the exact ad-level matcher on them.  The pages run
// this stage on the host CPU, so it is host C++ here, threaded over rows.
//
// Exact matcher: an ad passes when every attribute bit the user sets is set
// in the ad's rule words (eq 5 on one ad's rules) and one of the user's
// locations is in the ad's geo list (set membership); with no user locations
// the location part passes.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <thread>
#include <vector>

#include "gr_internal.h"

namespace {

gr_status post_fail(gr_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return gr::report(st, buf);
}

template <typename F>
void rows_parallel(int64_t n, int threads, F f) {
    if (n <= 0) return;
    if (threads <= 0) {
        const unsigned hc = std::thread::hardware_concurrency();
        threads = hc ? (int)std::min(hc, 64u) : 4;
    }
    threads = (int)std::max<int64_t>(1, std::min<int64_t>(threads, n / 256 + 1));
    if (threads == 1) {
        f(0, n);
        return;
    }
    std::vector<std::thread> th;
    const int64_t chunk = (n + threads - 1) / threads;
    for (int i = 0; i < threads; ++i) {
        const int64_t a = i * chunk, b = std::min(n, a + chunk);
        if (a >= b) break;
        th.emplace_back([=] { f(a, b); });
    }
    for (auto &t : th) t.join();
}

}  // namespace

struct gr_ad_index {
    int32_t L = 0, V = 0, bpt = 0, w_bm = 0;
    std::vector<uint64_t> key;        // distinct packed SIDs, sorted
    std::vector<int64_t> rank_of_row; // catalog row -> index into key
    std::vector<int64_t> ad_rank;     // ad -> key index of its SID
    std::vector<uint64_t> rules;      // [n_ads, w_bm]
    std::vector<int64_t> geo_off;     // [n_ads + 1]
    std::vector<int32_t> geo;         // per ad, sorted and distinct
    std::vector<int64_t> off;         // [n_keys + 1] ads of each SID (after finish)
    std::vector<int64_t> ads;
    bool finished = false;

    uint64_t pack(const int32_t *t) const {
        uint64_t k = 0;
        for (int l = 0; l < L; ++l) k = (k << bpt) | (uint64_t)t[l];
        return k;
    }
};

extern "C" {

gr_status gr_ad_index_create(const int32_t *sids, int64_t n_sids, int32_t sid_length,
                             int32_t vocab_size, int32_t w_bm, gr_ad_index **out) {
    if (!out) return post_fail(GR_E_INVALID, "gr_ad_index_create: out is NULL");
    *out = nullptr;
    if (n_sids < 1 || !sids) return post_fail(GR_E_INVALID, "gr_ad_index_create: no SIDs");
    if (sid_length < 1 || sid_length > 16 || vocab_size < 2 || w_bm < 1 || w_bm > gr::MAX_WBM)
        return post_fail(GR_E_INVALID, "gr_ad_index_create: L %d, V %d, w_bm %d invalid",
                         sid_length, vocab_size, w_bm);
    int bpt = 1;
    while ((1 << bpt) < vocab_size) ++bpt;
    if (bpt * sid_length > 64)
        return post_fail(GR_E_UNSUPPORTED, "gr_ad_index_create: L * ceil(log2 V) = %d exceeds 64",
                         bpt * sid_length);
    gr_ad_index *ix = new (std::nothrow) gr_ad_index;
    if (!ix) return post_fail(GR_E_NOMEM, "gr_ad_index_create: out of host memory");
    ix->L = sid_length;
    ix->V = vocab_size;
    ix->bpt = bpt;
    ix->w_bm = w_bm;
    try {
        std::vector<std::pair<uint64_t, int64_t>> kr((size_t)n_sids);
        for (int64_t r = 0; r < n_sids; ++r) {
            const int32_t *t = sids + r * sid_length;
            for (int l = 0; l < sid_length; ++l)
                if (t[l] < 0 || t[l] >= vocab_size) {
                    delete ix;
                    return post_fail(GR_E_INVALID, "gr_ad_index_create: SID %lld has token %d",
                                     (long long)r, t[l]);
                }
            kr[(size_t)r] = {ix->pack(t), r};
        }
        std::sort(kr.begin(), kr.end());
        ix->key.resize((size_t)n_sids);
        ix->rank_of_row.resize((size_t)n_sids);
        for (int64_t i = 0; i < n_sids; ++i) {
            if (i && kr[(size_t)i].first == kr[(size_t)i - 1].first) {
                delete ix;
                return post_fail(GR_E_INVALID, "gr_ad_index_create: SID rows %lld and %lld repeat",
                                 (long long)kr[(size_t)i - 1].second, (long long)kr[(size_t)i].second);
            }
            ix->key[(size_t)i] = kr[(size_t)i].first;
            ix->rank_of_row[(size_t)kr[(size_t)i].second] = i;
        }
        ix->geo_off.push_back(0);
    } catch (const std::bad_alloc &) {
        delete ix;
        return post_fail(GR_E_NOMEM, "gr_ad_index_create: out of host memory");
    }
    *out = ix;
    return GR_OK;
}

gr_status gr_ad_index_add_ads(gr_ad_index *ix, int64_t n_ads, const int64_t *ad_sid,
                              const uint64_t *rules, const int64_t *geo_offsets,
                              const int32_t *geo_ids) {
    if (!ix || ix->finished) return post_fail(GR_E_INVALID, "gr_ad_index_add_ads: no open index");
    if (n_ads < 0 || (n_ads > 0 && (!ad_sid || !rules || !geo_offsets)))
        return post_fail(GR_E_INVALID, "gr_ad_index_add_ads: null array");
    const int64_t n_rows = (int64_t)ix->rank_of_row.size();
    for (int64_t a = 0; a < n_ads; ++a) {
        if (ad_sid[a] < 0 || ad_sid[a] >= n_rows)
            return post_fail(GR_E_INVALID, "gr_ad_index_add_ads: ad %lld names SID row %lld",
                             (long long)a, (long long)ad_sid[a]);
        if (geo_offsets[a + 1] < geo_offsets[a] || (geo_offsets[a + 1] > geo_offsets[a] && !geo_ids))
            return post_fail(GR_E_INVALID, "gr_ad_index_add_ads: geo offsets of ad %lld", (long long)a);
    }
    try {
        for (int64_t a = 0; a < n_ads; ++a) {
            ix->ad_rank.push_back(ix->rank_of_row[(size_t)ad_sid[a]]);
            for (int w = 0; w < ix->w_bm; ++w) ix->rules.push_back(rules[a * ix->w_bm + w]);
            const size_t g0 = ix->geo.size();
            for (int64_t g = geo_offsets[a]; g < geo_offsets[a + 1]; ++g) ix->geo.push_back(geo_ids[g]);
            std::sort(ix->geo.begin() + (ptrdiff_t)g0, ix->geo.end());
            ix->geo.erase(std::unique(ix->geo.begin() + (ptrdiff_t)g0, ix->geo.end()), ix->geo.end());
            ix->geo_off.push_back((int64_t)ix->geo.size());
        }
    } catch (const std::bad_alloc &) {
        return post_fail(GR_E_NOMEM, "gr_ad_index_add_ads: out of host memory");
    }
    return GR_OK;
}

gr_status gr_ad_index_finish(gr_ad_index *ix) {
    if (!ix || ix->finished) return post_fail(GR_E_INVALID, "gr_ad_index_finish: no open index");
    try {
        const size_t nk = ix->key.size(), na = ix->ad_rank.size();
        ix->off.assign(nk + 1, 0);
        for (size_t a = 0; a < na; ++a) ++ix->off[(size_t)ix->ad_rank[a] + 1];
        for (size_t i = 0; i < nk; ++i) ix->off[i + 1] += ix->off[i];
        ix->ads.resize(na);
        std::vector<int64_t> pos(ix->off.begin(), ix->off.end() - 1);
        for (size_t a = 0; a < na; ++a) ix->ads[(size_t)pos[(size_t)ix->ad_rank[a]]++] = (int64_t)a;
    } catch (const std::bad_alloc &) {
        return post_fail(GR_E_NOMEM, "gr_ad_index_finish: out of host memory");
    }
    ix->finished = true;
    return GR_OK;
}

gr_status gr_post_filter(const gr_ad_index *ix, const int32_t *tokens, int64_t n_rows,
                         int64_t rows_per_request, const uint64_t *user_bm,
                         const int32_t *user_locs, int32_t n_loc, int64_t *counts,
                         int64_t *pass_ids, int64_t pass_cap, int32_t n_threads) {
    if (!ix || !ix->finished) return post_fail(GR_E_INVALID, "gr_post_filter: index not finished");
    if (n_rows < 0 || rows_per_request < 1 || n_loc < 0)
        return post_fail(GR_E_INVALID, "gr_post_filter: bad sizes");
    if (n_rows > 0 && (!tokens || !user_bm || !counts || (n_loc > 0 && !user_locs)))
        return post_fail(GR_E_INVALID, "gr_post_filter: null array");
    const int L = ix->L, wb = ix->w_bm;
    const int64_t n_req = (n_rows + rows_per_request - 1) / rows_per_request;
    // each request's locations, sorted, for membership tests
    std::vector<int32_t> locs;
    try {
        locs.assign(user_locs ? user_locs : (const int32_t *)nullptr,
                    user_locs ? user_locs + n_req * n_loc : (const int32_t *)nullptr);
    } catch (const std::bad_alloc &) {
        return post_fail(GR_E_NOMEM, "gr_post_filter: out of host memory");
    }
    for (int64_t b = 0; b < n_req; ++b)
        std::sort(locs.begin() + b * n_loc, locs.begin() + (b + 1) * n_loc);
    rows_parallel(n_rows, n_threads, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            int64_t *c = counts + r * 4;
            c[0] = c[1] = c[2] = c[3] = 0;
            const int32_t *t = tokens + r * L;
            bool ok = true;
            for (int l = 0; l < L; ++l) ok = ok && t[l] >= 0 && t[l] < ix->V;
            if (!ok) continue;   // a dead slot
            const uint64_t k = ix->pack(t);
            const auto it = std::lower_bound(ix->key.begin(), ix->key.end(), k);
            if (it == ix->key.end() || *it != k) continue;   // not a catalog SID
            const size_t kr = (size_t)(it - ix->key.begin());
            const int64_t b = r / rows_per_request;
            const uint64_t *u = user_bm + b * wb;
            const int32_t *lb = locs.data() + b * n_loc, *le = lb + n_loc;
            for (int64_t p = ix->off[kr]; p < ix->off[kr + 1]; ++p) {
                const int64_t a = ix->ads[(size_t)p];
                bool bm_ok = true;
                for (int w = 0; w < wb; ++w) bm_ok = bm_ok && (ix->rules[(size_t)(a * wb + w)] & u[w]) == u[w];
                bool geo_ok = n_loc == 0;
                for (int64_t g = ix->geo_off[(size_t)a]; g < ix->geo_off[(size_t)a + 1] && !geo_ok; ++g)
                    geo_ok = std::binary_search(lb, le, ix->geo[(size_t)g]);
                c[0] += 1;
                c[1] += bm_ok;
                c[2] += geo_ok;
                c[3] += bm_ok && geo_ok;
            }
        }
    });
    if (!pass_ids) return GR_OK;
    int64_t total = 0;
    for (int64_t r = 0; r < n_rows; ++r) total += counts[r * 4 + 3];
    if (total > pass_cap)
        return post_fail(GR_E_WORKSPACE, "gr_post_filter: %lld passing ads exceed pass_cap %lld",
                         (long long)total, (long long)pass_cap);
    int64_t o = 0;
    for (int64_t r = 0; r < n_rows; ++r) {   // ids of the passing ads, row by row
        if (!counts[r * 4 + 3]) continue;
        const int32_t *t = tokens + r * L;
        const size_t kr = (size_t)(std::lower_bound(ix->key.begin(), ix->key.end(), ix->pack(t)) -
                                   ix->key.begin());
        const int64_t b = r / rows_per_request;
        const uint64_t *u = user_bm + b * wb;
        const int32_t *lb = locs.data() + b * n_loc, *le = lb + n_loc;
        for (int64_t p = ix->off[kr]; p < ix->off[kr + 1]; ++p) {
            const int64_t a = ix->ads[(size_t)p];
            bool ok = true;
            for (int w = 0; w < wb; ++w) ok = ok && (ix->rules[(size_t)(a * wb + w)] & u[w]) == u[w];
            bool geo_ok = n_loc == 0;
            for (int64_t g = ix->geo_off[(size_t)a]; g < ix->geo_off[(size_t)a + 1] && !geo_ok; ++g)
                geo_ok = std::binary_search(lb, le, ix->geo[(size_t)g]);
            if (ok && geo_ok) pass_ids[o++] = a;
        }
    }
    return GR_OK;
}

void gr_ad_index_destroy(gr_ad_index *ix) { delete ix; }

}  // extern "C"
