/*
 * CPU oracle for the wide-beam SID decode step.
 *
 * TEST INFRASTRUCTURE ONLY: this file is compiled into oracle/_oracle.so and is
 * loaded by the tests, the smoke check and the benchmark's CPU-baseline leg.
 * It shares no code, header, table or constant with the GPU library.  Every
 * function is a plain, slow, literal rendering of the step it cites; loops run
 * in the order the definition reads, floating point is fp64 unless a step
 * says otherwise.
 *
 * Sources (GRACE, "Generative Recommender Acceleration Engine for Real-Time
 * Ads Retrieval", arXiv 2608.00938; the paper-archivist close reading and the
 * paperpeel English text):
 *   Section 4.1 eqs 1-3  (CD, TM, -inf masking of log-probabilities)
 *   Section 4.2 eqs 4-5  (bitmask union per trie node, packed containment test)
 *   Section 4.3 eqs 8-9  (Bloom containment test, ANY over user locations,
 *                         Bloom union per trie node)
 *   Section 3.1, 3.3     (log-prob accumulation, beam top-k, reorder)
 *   Section 5.1 eqs 10-14 and Appendix B (beam-as-query cross-attention)
 *   Section 5.2, 5.3     (short-prefix self-attention, paged block table;
 *                         here replaced by the dense per-row history that the
 *                         pages describe as the baseline being replaced)
 * The Bloom hash family is not given on the pages; this oracle uses the
 * reading stated next to orc_bloom_positions.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* O1: Bloom positions of one id.                                           */
/* Reading (pages silent): h = first output of SplitMix64 (Steele, Lea and  */
/* Flood 2014) started from state g; h1 = low 32 bits, h2 = high 32 bits | 1;*/
/* position i = (h1 + i*h2) mod w  (Kirsch-Mitzenmacher double hashing).    */
/* ------------------------------------------------------------------------ */
uint64_t orc_splitmix64_first(uint64_t state)
{
    uint64_t z = state + 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

void orc_bloom_positions(int64_t id, int w_bits, int k, uint32_t *out)
{
    uint64_t h = orc_splitmix64_first((uint64_t)id);
    uint64_t h1 = h & 0xFFFFFFFFULL;
    uint64_t h2 = (h >> 32) | 1ULL;
    for (int i = 0; i < k; i++)
        out[i] = (uint32_t)((h1 + (uint64_t)i * h2) % (uint64_t)w_bits);
}

/* bloom(l): the full w-bit filter of a single id (row of w/64 words). */
void orc_bloom_row(int64_t id, int w_bits, int k, uint64_t *row)
{
    uint32_t pos[64];
    memset(row, 0, sizeof(uint64_t) * (size_t)(w_bits / 64));
    orc_bloom_positions(id, w_bits, k, pos);
    for (int i = 0; i < k; i++)
        row[pos[i] / 64] |= 1ULL << (pos[i] % 64);
}

/* eq 8: contains(B, l) = [(bloom(l) AND B) == bloom(l)], on whole words. */
int orc_bloom_contains(const uint64_t *B, const uint64_t *bloom_l, int w_words)
{
    for (int i = 0; i < w_words; i++)
        if ((bloom_l[i] & B[i]) != bloom_l[i])
            return 0;
    return 1;
}

/* eq 5: (bitmask(p||v) AND bitmask(u)) == bitmask(u). */
int orc_bitmask_match(const uint64_t *node_bm, const uint64_t *user_bm, int w_words)
{
    for (int i = 0; i < w_words; i++)
        if ((node_bm[i] & user_bm[i]) != user_bm[i])
            return 0;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* O2: prefix tables.  For every level l = 1..L the distinct length-l       */
/* prefixes of catalog SIDs, sorted lexicographically, each with            */
/* bitmask(p) = OR of its ads' rules (eq 4) and bloom(p) = OR of its ads'   */
/* Bloom filters (eq 9).  Built from the catalog and the ad list directly.  */
/* ------------------------------------------------------------------------ */
typedef struct {
    int L, V, w_bm, w_bl, bloom_bits, bloom_k;
    int64_t n_sids;
    int32_t *sids;       /* [n_sids, L] copy                                */
    uint64_t *leaf_bm;   /* [n_sids, w_bm]: OR over the SID's own ads        */
    uint64_t *leaf_bl;   /* [n_sids, w_bl]                                  */
    int64_t n[17];       /* prefixes per level                              */
    int32_t *pfx[17];    /* [n_l, l]                                        */
    uint64_t *bm[17];    /* [n_l, w_bm]                                     */
    uint64_t *bl[17];    /* [n_l, w_bl]                                     */
    int finished;
} orc_index;

orc_index *orc_index_create(int L, int V, int64_t n_sids, const int32_t *sids,
                            int w_bm, int bloom_bits, int bloom_k)
{
    if (L < 1 || L > 16) return NULL;
    orc_index *ix = (orc_index *)calloc(1, sizeof(orc_index));
    ix->L = L; ix->V = V; ix->w_bm = w_bm;
    ix->bloom_bits = bloom_bits; ix->bloom_k = bloom_k;
    ix->w_bl = bloom_bits / 64;
    ix->n_sids = n_sids;
    ix->sids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_sids * L);
    memcpy(ix->sids, sids, sizeof(int32_t) * (size_t)n_sids * L);
    ix->leaf_bm = (uint64_t *)calloc((size_t)n_sids * (w_bm ? w_bm : 1), sizeof(uint64_t));
    ix->leaf_bl = (uint64_t *)calloc((size_t)n_sids * (ix->w_bl ? ix->w_bl : 1), sizeof(uint64_t));
    return ix;
}

/* Fold a batch of ads into their SIDs' own unions. */
void orc_index_add_ads(orc_index *ix, int64_t n_ads, const int64_t *ad_sid,
                       const uint64_t *rules, const int64_t *geo_off,
                       const int32_t *geo_ids)
{
    for (int64_t a = 0; a < n_ads; a++) {
        int64_t s = ad_sid[a];
        for (int w = 0; w < ix->w_bm; w++)
            ix->leaf_bm[s * ix->w_bm + w] |= rules[a * ix->w_bm + w];
        if (ix->w_bl) {
            /* bloom(a) = OR of bloom(g) over the ad's geo ids: set each id's bits */
            uint32_t pos[64];
            for (int64_t j = geo_off[a]; j < geo_off[a + 1]; j++) {
                orc_bloom_positions(geo_ids[j], ix->bloom_bits, ix->bloom_k, pos);
                for (int i = 0; i < ix->bloom_k; i++)
                    ix->leaf_bl[s * ix->w_bl + pos[i] / 64] |= 1ULL << (pos[i] % 64);
            }
        }
    }
}

static const orc_index *g_sort_ix;
static int cmp_sid(const void *a, const void *b)
{
    int64_t i = *(const int64_t *)a, j = *(const int64_t *)b;
    const int32_t *x = g_sort_ix->sids + i * g_sort_ix->L;
    const int32_t *y = g_sort_ix->sids + j * g_sort_ix->L;
    for (int l = 0; l < g_sort_ix->L; l++) {
        if (x[l] != y[l]) return x[l] < y[l] ? -1 : 1;
    }
    return (i > j) - (i < j);
}

void orc_index_finish(orc_index *ix)
{
    int L = ix->L;
    int64_t N = ix->n_sids;
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    for (int64_t i = 0; i < N; i++) order[i] = i;
    g_sort_ix = ix;
    qsort(order, (size_t)N, sizeof(int64_t), cmp_sid);
    for (int l = 1; l <= L; l++) {
        /* count distinct length-l prefixes along the sorted order */
        int64_t n = 0;
        for (int64_t r = 0; r < N; r++) {
            const int32_t *cur = ix->sids + order[r] * L;
            if (r == 0 || memcmp(cur, ix->sids + order[r - 1] * L, sizeof(int32_t) * l) != 0)
                n++;
        }
        ix->n[l] = n;
        ix->pfx[l] = (int32_t *)malloc(sizeof(int32_t) * (size_t)n * l);
        ix->bm[l] = (uint64_t *)calloc((size_t)n * (ix->w_bm ? ix->w_bm : 1), sizeof(uint64_t));
        ix->bl[l] = (uint64_t *)calloc((size_t)n * (ix->w_bl ? ix->w_bl : 1), sizeof(uint64_t));
        int64_t p = -1;
        for (int64_t r = 0; r < N; r++) {
            int64_t s = order[r];
            const int32_t *cur = ix->sids + s * L;
            if (r == 0 || memcmp(cur, ix->sids + order[r - 1] * L, sizeof(int32_t) * l) != 0) {
                p++;
                memcpy(ix->pfx[l] + p * l, cur, sizeof(int32_t) * l);
            }
            for (int w = 0; w < ix->w_bm; w++)
                ix->bm[l][p * ix->w_bm + w] |= ix->leaf_bm[s * ix->w_bm + w];
            for (int w = 0; w < ix->w_bl; w++)
                ix->bl[l][p * ix->w_bl + w] |= ix->leaf_bl[s * ix->w_bl + w];
        }
    }
    ix->n[0] = 1;
    free(order);
    ix->finished = 1;
}

void orc_index_destroy(orc_index *ix)
{
    if (!ix) return;
    for (int l = 0; l <= 16; l++) { free(ix->pfx[l]); free(ix->bm[l]); free(ix->bl[l]); }
    free(ix->sids); free(ix->leaf_bm); free(ix->leaf_bl);
    free(ix);
}

int64_t orc_index_count(const orc_index *ix, int level) { return ix->n[level]; }

/* Position of a length-l prefix in level l's sorted table, or -1. */
int64_t orc_index_find(const orc_index *ix, const int32_t *prefix, int l)
{
    if (l == 0) return 0;
    int64_t lo = 0, hi = ix->n[l] - 1;
    while (lo <= hi) {
        int64_t mid = lo + (hi - lo) / 2;
        const int32_t *p = ix->pfx[l] + mid * l;
        int c = 0;
        for (int i = 0; i < l && c == 0; i++)
            c = (p[i] < prefix[i]) ? -1 : (p[i] > prefix[i]) ? 1 : 0;
        if (c == 0) return mid;
        if (c < 0) lo = mid + 1; else hi = mid - 1;
    }
    return -1;
}

/* Copy out a level's matcher rows (for checking a built index against it). */
void orc_index_rows(const orc_index *ix, int l, int32_t *pfx, uint64_t *bm, uint64_t *bl)
{
    int64_t n = ix->n[l];
    if (pfx) memcpy(pfx, ix->pfx[l], sizeof(int32_t) * (size_t)n * l);
    if (bm && ix->w_bm) memcpy(bm, ix->bm[l], sizeof(uint64_t) * (size_t)n * ix->w_bm);
    if (bl && ix->w_bl) memcpy(bl, ix->bl[l], sizeof(uint64_t) * (size_t)n * ix->w_bl);
}

/* ------------------------------------------------------------------------ */
/* O3-O5: the CD and TM masks of one beam row (eqs 1, 2, 5, 8).             */
/* prefix: the row's t tokens; t < 0 marks a dead row (all tokens masked).  */
/* user_bm [w_bm]; user_blooms [n_loc, w_bl]: bloom(l) of each user         */
/* location (orc_bloom_row).  mask: ceil(V/64) words.                       */
/* Returns the number of tokens kept.                                       */
/* ------------------------------------------------------------------------ */
int orc_mask_row(const orc_index *ix, const int32_t *prefix, int t,
                 const uint64_t *user_bm, const uint64_t *user_blooms, int n_loc,
                 uint64_t *mask)
{
    int V = ix->V, words = (V + 63) / 64, kept = 0;
    memset(mask, 0, sizeof(uint64_t) * (size_t)words);
    if (t < 0 || t >= ix->L) return 0;
    int32_t child[17];
    for (int i = 0; i < t; i++) child[i] = prefix[i];
    for (int v = 0; v < V; v++) {
        child[t] = v;
        int64_t c = orc_index_find(ix, child, t + 1);
        int cd = (c >= 0);                                  /* eq 1 */
        if (!cd) continue;
        int bm_ok = orc_bitmask_match(ix->bm[t + 1] + c * ix->w_bm, user_bm, ix->w_bm);
        int bl_ok = 1;
        if (ix->w_bl) {                                     /* eq 8, ANY of locations */
            bl_ok = 0;
            for (int j = 0; j < n_loc && !bl_ok; j++)
                bl_ok = orc_bloom_contains(ix->bl[t + 1] + c * ix->w_bl,
                                           user_blooms + (size_t)j * ix->w_bl, ix->w_bl);
        }
        if (bm_ok && bl_ok) {                               /* CD * TM = 1 */
            mask[v / 64] |= 1ULL << (v % 64);
            kept++;
        }
    }
    return kept;
}

/* ------------------------------------------------------------------------ */
/* O6: log-softmax over the full vocabulary, fp64.                          */
/* ------------------------------------------------------------------------ */
void orc_log_softmax(const double *x, int V, double *lp)
{
    double mx = -INFINITY;
    for (int v = 0; v < V; v++) if (x[v] > mx) mx = x[v];
    double s = 0.0;
    for (int v = 0; v < V; v++) s += exp(x[v] - mx);
    double lse = mx + log(s);
    for (int v = 0; v < V; v++) lp[v] = x[v] - lse;
}

/* ------------------------------------------------------------------------ */
/* O8: per-request top-k over flat candidates f = m*V + v.                  */
/* Order: score descending, then f ascending; -inf entries are not          */
/* candidates.  Returns the number selected (<= k).                         */
/* ------------------------------------------------------------------------ */
typedef struct { float s; uint32_t f; } orc_cand;
static int cmp_cand(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->s != y->s) return x->s > y->s ? -1 : 1;
    return (x->f > y->f) - (x->f < y->f);
}

int64_t orc_topk(const float *scores, int64_t n, int64_t k, uint32_t *sel_f, float *sel_s)
{
    orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(n ? n : 1));
    int64_t m = 0;
    for (int64_t f = 0; f < n; f++)
        if (isfinite(scores[f])) { c[m].s = scores[f]; c[m].f = (uint32_t)f; m++; }
    qsort(c, (size_t)m, sizeof(orc_cand), cmp_cand);
    int64_t out = m < k ? m : k;
    for (int64_t i = 0; i < out; i++) { sel_f[i] = c[i].f; sel_s[i] = c[i].s; }
    free(c);
    return out;
}

/* ------------------------------------------------------------------------ */
/* O10a: cross-attention, beam-as-query (eqs 11-14).  Row r = b*M + m reads */
/* request b's K, V.  q [R,H,d], K/V [B,H,T,d], out [R,H,d]; scale 1/sqrt(d)*/
/* ------------------------------------------------------------------------ */
void orc_cross_attn(const double *q, const double *K, const double *Vv,
                    int B, int M, int H, int T, int d, double *out)
{
    double scale = 1.0 / sqrt((double)d);
    int64_t R = (int64_t)B * M;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        int64_t b = r / M;
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        for (int h = 0; h < H; h++) {
            const double *qr = q + (r * H + h) * d;
            const double *Kb = K + ((b * H + h) * (int64_t)T) * d;
            const double *Vb = Vv + ((b * H + h) * (int64_t)T) * d;
            double mx = -INFINITY;
            for (int tau = 0; tau < T; tau++) {
                double acc = 0.0;
                for (int i = 0; i < d; i++) acc += qr[i] * Kb[tau * d + i];
                s[tau] = acc * scale;
                if (s[tau] > mx) mx = s[tau];
            }
            double z = 0.0;
            for (int tau = 0; tau < T; tau++) { s[tau] = exp(s[tau] - mx); z += s[tau]; }
            double *o = out + (r * H + h) * d;
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int tau = 0; tau < T; tau++) acc += s[tau] * Vb[tau * d + i];
                o[i] = acc / z;
            }
        }
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* O10b: self-attention over each row's own dense prefix history.           */
/* q [R,H,d]; hk/hv [R,T,H,d]; valid [R,T] (0 = position excluded).         */
/* Each row attends only to its own positions (the block-diagonal mask of   */
/* Section 5.2).  A row with no valid position gets zeros.                  */
/* ------------------------------------------------------------------------ */
void orc_self_attn(const double *q, const double *hk, const double *hv,
                   const uint8_t *valid, int64_t R, int T, int H, int d, double *out)
{
    double scale = 1.0 / sqrt((double)d);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        double s[64];
        for (int h = 0; h < H; h++) {
            const double *qr = q + (r * H + h) * d;
            double mx = -INFINITY;
            for (int j = 0; j < T; j++) {
                if (!valid[r * T + j]) continue;
                const double *kr = hk + ((r * T + j) * H + h) * d;
                double acc = 0.0;
                for (int i = 0; i < d; i++) acc += qr[i] * kr[i];
                s[j] = acc * scale;
                if (s[j] > mx) mx = s[j];
            }
            double z = 0.0;
            for (int j = 0; j < T; j++) {
                if (!valid[r * T + j]) continue;
                s[j] = exp(s[j] - mx); z += s[j];
            }
            double *o = out + (r * H + h) * d;
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int j = 0; j < T; j++) {
                    if (!valid[r * T + j]) continue;
                    acc += s[j] * hv[((r * T + j) * H + h) * d + i];
                }
                o[i] = z > 0.0 ? acc / z : 0.0;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* F2: joint attention over the request's context and the row's own beam    */
/* prefix, one softmax over the concatenated key sequence (the shared-      */
/* prefix beam attention of the Meituan engine article; GR-Inference's      */
/* GR-Decode-Attention, whose K1 / K2 partial results its K3 merges with a  */
/* log-sum-exp, computes the same thing).  Row r = b*M + m.                 */
/* q [R,H,d]; K/V [B,H,T,d]; hk/hv [R,Tb,H,d]; valid [R,Tb] (0 = excluded). */
/* out [R,H,d]; scale 1/sqrt(d).                                            */
/* ------------------------------------------------------------------------ */
void orc_joint_attn(const double *q, const double *K, const double *Vv,
                    const double *hk, const double *hv, const uint8_t *valid,
                    int B, int M, int H, int T, int Tb, int d, double *out)
{
    double scale = 1.0 / sqrt((double)d);
    int64_t R = (int64_t)B * M;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        int64_t b = r / M;
        double *s = (double *)malloc(sizeof(double) * (size_t)(T + Tb));
        for (int h = 0; h < H; h++) {
            const double *qr = q + (r * H + h) * d;
            const double *Kb = K + ((b * H + h) * (int64_t)T) * d;
            const double *Vb = Vv + ((b * H + h) * (int64_t)T) * d;
            /* scores: context positions 0..T-1, then beam positions T..T+Tb-1 */
            double mx = -INFINITY;
            for (int j = 0; j < T + Tb; j++) {
                if (j >= T && !valid[r * Tb + (j - T)]) continue;
                const double *kr = j < T ? Kb + (int64_t)j * d : hk + ((r * Tb + (j - T)) * H + h) * d;
                double acc = 0.0;
                for (int i = 0; i < d; i++) acc += qr[i] * kr[i];
                s[j] = acc * scale;
                if (s[j] > mx) mx = s[j];
            }
            double z = 0.0;
            for (int j = 0; j < T + Tb; j++) {
                if (j >= T && !valid[r * Tb + (j - T)]) continue;
                s[j] = exp(s[j] - mx);
                z += s[j];
            }
            double *o = out + (r * H + h) * d;
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int j = 0; j < T + Tb; j++) {
                    if (j >= T && !valid[r * Tb + (j - T)]) continue;
                    const double *vr = j < T ? Vb + (int64_t)j * d : hv + ((r * Tb + (j - T)) * H + h) * d;
                    acc += s[j] * vr[i];
                }
                o[i] = acc / z;
            }
        }
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* Threads of the loops over rows above (timing only: each row's arithmetic */
/* is the same whatever the count).                                          */
/* ------------------------------------------------------------------------ */
void orc_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

int orc_get_threads(void)
{
    return omp_get_max_threads();
}


/* ------------------------------------------------------------------------ */
/* Large catalogs: matcher unions of sampled prefixes (eqs 4 and 9), built  */
/* from the catalog and the ad stream directly.  For each level l the       */
/* caller names the prefixes to sample by their base-V code                 */
/* (t_1 * V^(l-1) + ... + t_l), sorted; every ad whose SID starts with a     */
/* sampled prefix ORs its rule words and the Bloom positions of its geo ids  */
/* into that prefix's rows.  Ads can be added in any number of calls.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    int L, V, w_bm, w_bl, bloom_bits, bloom_k;
    const int32_t *sids;     /* [n_sids, L], the caller's (kept alive by it) */
    int64_t n_sids;
    int64_t n[17];           /* sampled prefixes per level                   */
    int64_t *code[17];       /* [n_l] sorted base-V codes                    */
    uint64_t *bm[17];        /* [n_l, w_bm]                                  */
    uint64_t *bl[17];        /* [n_l, w_bl]                                  */
} orc_usample;

orc_usample *orc_usample_create(int L, int V, int w_bm, int bloom_bits, int bloom_k,
                                const int32_t *sids, int64_t n_sids)
{
    if (L < 1 || L > 16) return NULL;
    orc_usample *u = (orc_usample *)calloc(1, sizeof(orc_usample));
    u->L = L; u->V = V; u->w_bm = w_bm; u->bloom_bits = bloom_bits;
    u->bloom_k = bloom_k; u->w_bl = bloom_bits / 64;
    u->sids = sids; u->n_sids = n_sids;
    return u;
}

void orc_usample_destroy(orc_usample *u)
{
    if (!u) return;
    for (int l = 0; l <= 16; l++) { free(u->code[l]); free(u->bm[l]); free(u->bl[l]); }
    free(u);
}

void orc_usample_set_level(orc_usample *u, int level, const int64_t *codes, int64_t n)
{
    free(u->code[level]); free(u->bm[level]); free(u->bl[level]);
    u->n[level] = n;
    u->code[level] = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
    memcpy(u->code[level], codes, sizeof(int64_t) * (size_t)n);
    u->bm[level] = (uint64_t *)calloc((size_t)(n ? n : 1) * u->w_bm, sizeof(uint64_t));
    u->bl[level] = (uint64_t *)calloc((size_t)(n ? n : 1) * (u->w_bl ? u->w_bl : 1),
                                      sizeof(uint64_t));
}

static int64_t find_code(const int64_t *a, int64_t n, int64_t key)
{
    int64_t lo = 0, hi = n;            /* plain binary search */
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    return (lo < n && a[lo] == key) ? lo : -1;
}

void orc_usample_add_ads(orc_usample *u, int64_t n_ads, const int64_t *ad_sid,
                         const uint64_t *rules, const int64_t *geo_off, const int32_t *geo_ids)
{
    const int L = u->L, wbm = u->w_bm, wbl = u->w_bl;
    const int nt = omp_get_max_threads();
    /* each thread ORs into rows of its own; the rows are merged at the end */
    int64_t tot_bm = 0, tot_bl = 0, base_bm[17], base_bl[17];
    for (int l = 1; l <= L; l++) {
        base_bm[l] = tot_bm; base_bl[l] = tot_bl;
        tot_bm += u->n[l] * wbm; tot_bl += u->n[l] * wbl;
    }
    uint64_t *pbm = (uint64_t *)calloc((size_t)nt * (tot_bm ? tot_bm : 1), sizeof(uint64_t));
    uint64_t *pbl = (uint64_t *)calloc((size_t)nt * (tot_bl ? tot_bl : 1), sizeof(uint64_t));
    #pragma omp parallel num_threads(nt)
    {
        const int th = omp_get_thread_num();
        uint64_t *mbm = pbm + (size_t)th * tot_bm;
        uint64_t *mbl = pbl + (size_t)th * tot_bl;
        uint32_t pos[64];
        int64_t hit[17];
        #pragma omp for schedule(dynamic, 4096)
        for (int64_t a = 0; a < n_ads; a++) {
            const int32_t *sid = u->sids + (size_t)ad_sid[a] * L;
            int64_t code = 0;
            int any = 0;
            for (int l = 1; l <= L; l++) {
                code = code * u->V + sid[l - 1];
                hit[l] = u->n[l] ? find_code(u->code[l], u->n[l], code) : -1;
                if (hit[l] >= 0) any = 1;
            }
            if (!any) continue;
            for (int l = 1; l <= L; l++) {
                if (hit[l] < 0) continue;
                uint64_t *r = mbm + base_bm[l] + hit[l] * wbm;
                for (int q = 0; q < wbm; q++) r[q] |= rules[a * wbm + q];
            }
            if (!wbl) continue;
            for (int64_t j = geo_off[a]; j < geo_off[a + 1]; j++) {
                orc_bloom_positions(geo_ids[j], u->bloom_bits, u->bloom_k, pos);
                for (int l = 1; l <= L; l++) {
                    if (hit[l] < 0) continue;
                    uint64_t *r = mbl + base_bl[l] + hit[l] * wbl;
                    for (int i = 0; i < u->bloom_k; i++) r[pos[i] / 64] |= 1ULL << (pos[i] % 64);
                }
            }
        }
    }
    for (int l = 1; l <= L; l++) {
        const int64_t nbm = u->n[l] * wbm, nbl = u->n[l] * wbl;
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < nbm; i++)
            for (int th = 0; th < nt; th++) u->bm[l][i] |= pbm[(size_t)th * tot_bm + base_bm[l] + i];
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < nbl; i++)
            for (int th = 0; th < nt; th++) u->bl[l][i] |= pbl[(size_t)th * tot_bl + base_bl[l] + i];
    }
    free(pbm);
    free(pbl);
}

void orc_usample_rows(const orc_usample *u, int level, uint64_t *bm, uint64_t *bl)
{
    memcpy(bm, u->bm[level], sizeof(uint64_t) * (size_t)u->n[level] * u->w_bm);
    if (u->w_bl) memcpy(bl, u->bl[level], sizeof(uint64_t) * (size_t)u->n[level] * u->w_bl);
}

/* ------------------------------------------------------------------------ */
/* Appendix A Lookup over a trie given as data (the Appendix A arrays of an */
/* index built elsewhere): follow the row's prefix from the root through    */
/* the child entries of each node (a linear scan for the token), then keep  */
/* token tok[e] of each child entry e of the reached node when eq 5 holds   */
/* for its bitmask row and, with Bloom rows, eq 8 holds for one of the      */
/* user's locations.  t < 0, or a prefix the trie does not hold, gives an   */
/* all-zero mask (a dead row).  Returns the number of kept tokens.          */
/* ------------------------------------------------------------------------ */
int orc_mask_row_csr(const int32_t *off, const int32_t *child, const int16_t *tok,
                     const int32_t *bmi, const int32_t *bli, const uint64_t *bm_tab, int w_bm,
                     const uint64_t *bl_tab, int w_bl, int V, const int32_t *prefix, int t,
                     const uint64_t *user_bm, const uint64_t *user_blooms, int n_loc,
                     uint64_t *out)
{
    memset(out, 0, sizeof(uint64_t) * (size_t)((V + 63) / 64));
    if (t < 0) return 0;
    int64_t node = 0;
    for (int j = 0; j < t; j++) {
        int64_t next = -1;
        for (int32_t e = off[node]; e < off[node + 1]; e++)
            if (tok[e] == prefix[j]) { next = child[e]; break; }
        if (next < 0) return 0;
        node = next;
    }
    int kept = 0;
    for (int32_t e = off[node]; e < off[node + 1]; e++) {
        if (!orc_bitmask_match(bm_tab + (size_t)bmi[e] * w_bm, user_bm, w_bm)) continue;
        int bl_ok = 1;
        if (w_bl) {
            bl_ok = 0;
            const uint64_t *row = bl_tab + (size_t)bli[e] * w_bl;
            for (int l = 0; l < n_loc && !bl_ok; l++)
                bl_ok = orc_bloom_contains(row, user_blooms + (size_t)l * w_bl, w_bl);
        }
        if (!bl_ok) continue;
        out[tok[e] / 64] |= 1ULL << (tok[e] % 64);
        kept++;
    }
    return kept;
}
