// CD + GTM constrain, full-vocabulary log-softmax, score accumulation,
// per-request top-k and beam reorder on gfx950.
//
// GRACE Section 3.1 (decode loop), Section 3.3 (beam top-k, dynamic widths,
// paged beam rearrangement), Section 4.1 eqs 1-3 (CD, TM, -inf masking),
// Section 4.2 eq 5 (packed bitmask test), Section 4.3 eq 8 (Bloom test, ANY
// of the user's locations), Section 4.4 / Appendix A (CSR Lookup over a
// node's child entries with deduplicated matcher rows).
//
// Two launches on one stream (gr_constrain, then gr_topk_reorder):
//   k_expand   a workgroup takes up to 32 beam rows of one request: the
//              request's bound U_b (best live parent score; every candidate
//              is <= U_b since log-probs are <= 0), each row's log-sum-exp
//              over all V logits, eqs 5 and 8 for every child of a node with
//              a bit-sliced matcher block, then the other rows' child
//              entries, two per thread per round: eq 5 from the
//              entry-ordered bitmask row, eq 8 for the entries still in
//              (their Bloom rows tested by all wavefronts from the round's
//              list, the owner thread emitting the entries that pass); the
//              rows' logits stay in LDS when they fit.  Survivors go to the
//              workgroup's own
//              segment and a 2048-bin histogram of U_b - score, merged into
//              the request's histogram.
//   k_select   one workgroup per request: the bin holding the k-th best
//              survivor from the histogram (which it clears again), every
//              survivor of a better bin, the threshold bin resolved exactly
//              (rank by counting, bitonic sort, or an MSB radix select over
//              global memory when it is large), the winners ordered by
//              (score desc, flat index asc), and the reorder writes parent /
//              token / child node / score and the token and block-table rows
//              of the new beams.
#include <algorithm>
#include <mutex>

#include "gr_device.h"
#include "gr_internal.h"

namespace gr {
namespace {

constexpr int EXP_WAVES = 4;
constexpr int EXP_THREADS = 64 * EXP_WAVES;
constexpr int STAGE_BYTES = 4352;     // Bloom rows staged per wavefront (8 x 4096 bits)
constexpr int NQ = 16;                // 8-byte staging registers per lane (wide rows)
constexpr int MAX_KP = 8;             // probes per location held in registers (more: LDS)
constexpr int NM_KP = 5;              // probes per location of the node-major pass (registers only)
constexpr int NM_SW = 8;              // node-major survivor words whose loads are in flight together
constexpr int NM_LG = 2;              // node-major 16-byte logit pieces per lane loaded up front
constexpr int LG_BYTES = 8192;        // bf16 logit rows an expand workgroup keeps in LDS
constexpr int BUF_DWORD3 = 0x00020000;  // buffer descriptor word 3 for gfx9 raw loads
constexpr int SEL_THREADS = 1024;
constexpr int BND_CAP = 2048;         // threshold-bin entries buffered in LDS
constexpr uint32_t BIN_SCAN_MIN = 16 * SEL_THREADS;   // survivors from which select reads bins first
constexpr uint32_t CAND_CAP = 4096;   // candidates (bins up to the threshold) listed in LDS

struct TailParams {
    const int32_t *off;
    const int32_t *child;
    const int16_t *tok;
    const int32_t *bmi;
    const int32_t *bli;
    const uint64_t *bm_tab;
    const uint64_t *bl_tab;
    const int64_t *nslice;      // bit-sliced Bloom block of each node (-1: none)
    const uint64_t *slice_tab;
    int w_bm, w_bl, bloom_k, bloom_bits;
    int64_t num_nodes;
    int B, M_in, V, k_out, t, L, n_loc;
    const uint64_t *user_bm;
    const uint32_t *user_probes;
    const void *logits;
    const int32_t *node_in;
    const float *acc_in;
    const int32_t *tokens_in;
    const int32_t *table_in;
    int32_t *parent_out, *token_out, *node_out;
    float *acc_out;
    int32_t *tokens_out, *table_out;
    uint64_t *dbg_mask;
    float *dbg_scores;
    uint32_t *segcnt;   // survivors of each expand workgroup [B, gx]
    uint32_t *hist;
    uint64_t *skey;     // survivor segments [B, gx, seg_cap]
    int32_t *schild;
    uint16_t *sbin;     // each survivor's histogram bin (0xFFFF: a pad)
    int64_t seg_cap;
    int gx;
    // expand launch shape
    int rows_wg;        // beam rows per workgroup
    int G;              // Bloom rows staged per sub-round
    int log2_wq;        // log2 of the 8-byte words per Bloom row
    int stage_dw;       // staging dwords per wavefront
    int mask_words;     // per-row mask words kept in LDS (debug outputs), else 0
    int tpr, log2_tpr;  // threads per row of the log-sum-exp
    int wmax;           // pass-vector words per row (bit-sliced rows), else 0
    int vec_logits;     // bf16 logits readable 8 at a time (V % 8 == 0, 16-byte base)
    const uint64_t *ent_bm;   // entry-ordered bitmask rows (null: gather through bmi)
    int vec_rows;             // token / block-table rows movable as 16-byte pieces
    const int32_t *kw_off, *kw_bmi, *kw_bli;   // k-way partitions (null: one union per entry)
    int lds_lg;         // the rows' bf16 logits are kept in LDS by the log-sum-exp pass
    // Node-major pass at the step after the root (k_expand_nm): the rows of
    // root children 1..n_nm that the inverse map names are tested there.
    int n_nm;           // root children taken node-major this call (0: none)
    int map_write;      // k_select records each output row's root child in inv
    int n_root;         // the root's children are nodes 1..n_root
    int32_t *inv;       // [B, V]: beam row of request b at root child v + 1
    uint32_t *segback;  // [MAX_B, NM_MAX_GX]: node-major survivors at the back of each segment
    uint32_t *cut;      // [MAX_B, NCUT]: survivors counted at or below the cutoff bins
    int nm_wave_dw;     // LDS dwords per node-major wavefront
    int nm_wgs;         // node-major workgroups at the front of k_expand's grid
};

// Lane-wise minimum of two pairs of unsigned 16-bit values.
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Bin of a candidate score below the request bound U (monotone
// non-increasing in the score: a better score never lands in a later bin).
__device__ __forceinline__ int score_bin(float s, float U) {
    float d = (U - s) * BIN_SCALE;
    if (!(d > 0.0f)) return 0;
    return d >= (float)(NBINS - 1) ? NBINS - 1 : (int)d;
}

// Row m of request b at node `node` is the node-major pass's (k_expand_nm):
// the node is a root child with a bit-sliced block and the inverse map names
// row m for it.  k_expand and k_expand_nm both decide by this test.
__device__ __forceinline__ bool nm_covered(const TailParams &p, int b, int m, int node,
                                           int64_t blk) {
    return p.n_nm && node >= 1 && node <= p.n_nm && blk >= 0 &&
           p.inv[(size_t)b * p.V + node - 1] == m;
}

// 64-bit selection key: higher = better; score first, then lower flat index.
__device__ __forceinline__ uint64_t make_key(float s, uint32_t f) {
    return ((uint64_t)f32_ord(s) << 32) | (uint64_t)(0xFFFFFFFFu - f);
}
__device__ __forceinline__ float key_score(uint64_t k) { return f32_unord((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_flat(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

// Partial max of the live parent scores of request b held by this thread;
// the caller reduces it over the workgroup.  Every candidate score of the
// request is at most the full max (log-probabilities are <= 0), so the score
// histogram bins hang below it.  The same rows and the same max (exact in
// floating point) give expand and select the same bound.
// The first chunk's loads of bound_part, issued early: the reduction
// (bound_finish) runs after other loads, so they share a round trip.
struct BoundLoads {
    int32_t n4[4];
    float a4[4];
};
__device__ __forceinline__ BoundLoads bound_load(const TailParams &p, int b) {
    BoundLoads o;
    const int32_t *nd = p.node_in + (size_t)b * p.M_in;
    const float *ac = p.acc_in + (size_t)b * p.M_in;
    const int nt = blockDim.x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = (int)threadIdx.x + q * nt;
        o.n4[q] = m < p.M_in ? nd[m] : -1;
        o.a4[q] = m < p.M_in ? ac[m] : -INFINITY;
    }
    return o;
}
__device__ __forceinline__ float bound_finish(const TailParams &p, int b, const BoundLoads &f) {
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (f.n4[q] >= 0 && f.n4[q] < p.num_nodes) mx = fmaxf(mx, f.a4[q]);
    const int32_t *nd = p.node_in + (size_t)b * p.M_in;
    const float *ac = p.acc_in + (size_t)b * p.M_in;
    const int nt = blockDim.x;
    for (int m = (int)threadIdx.x + 4 * nt; m < p.M_in; m += nt) {   // rows past the first chunk
        const int32_t n = nd[m];
        if (n >= 0 && n < p.num_nodes) mx = fmaxf(mx, ac[m]);
    }
    return wave_max(mx);
}

__device__ __forceinline__ float bound_part(const TailParams &p, int b) {
    float mx = -INFINITY;
    const int32_t *nd = p.node_in + (size_t)b * p.M_in;
    const float *ac = p.acc_in + (size_t)b * p.M_in;
    const int nt = blockDim.x;
    for (int m0 = threadIdx.x; m0 < p.M_in; m0 += 4 * nt) {
        int32_t n4[4];
        float a4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {   // every load first, then the compares
            const int m = m0 + q * nt;
            n4[q] = m < p.M_in ? nd[m] : -1;
            a4[q] = m < p.M_in ? ac[m] : -INFINITY;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (n4[q] >= 0 && n4[q] < p.num_nodes) mx = fmaxf(mx, a4[q]);
    }
    return wave_max(mx);
}

template <bool BF16>
__device__ __forceinline__ float logit_at(const void *logits, size_t idx) {
    if (BF16) return bf16_to_f32(((const uint16_t *)logits)[idx]);
    return ((const float *)logits)[idx];
}

// Running (max, sum of exp(x - max)) of one more logit.
__device__ __forceinline__ void lse_push(float x, float &m, float &s) {
    if (x > m) {
        s = s * __expf(m - x) + 1.0f;
        m = x;
    } else {
        s += __expf(x - m);
    }
}

// Set bits of a ballot in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// OR / AND of a 64-bit value over the wavefront (all lanes active)
__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
    return (uint64_t)wave_or32((uint32_t)v) | ((uint64_t)wave_or32((uint32_t)(v >> 32)) << 32);
}

__device__ __forceinline__ uint64_t wave_and64(uint64_t v) {
    return (uint64_t)wave_and32((uint32_t)v) | ((uint64_t)wave_and32((uint32_t)(v >> 32)) << 32);
}

// Four words w0 .. w0 + 3 of a bit-sliced column, loaded unconditionally
// (16 bytes at a time when the column width wc is even: blocks start
// 512-byte aligned).  Words past the column belong to the next positions or
// to the table's 4-word tail pad; callers ignore them.
__device__ __forceinline__ void col4(const uint64_t *col, bool even, uint64_t w[4]) {
    if (even) {
        const uint4 u = *(const uint4 *)col;
        const uint4 u2 = *(const uint4 *)(col + 2);
        w[0] = (uint64_t)u.x | ((uint64_t)u.y << 32);
        w[1] = (uint64_t)u.z | ((uint64_t)u.w << 32);
        w[2] = (uint64_t)u2.x | ((uint64_t)u2.y << 32);
        w[3] = (uint64_t)u2.z | ((uint64_t)u2.w << 32);
    } else {
        w[0] = col[0];
        w[1] = col[1];
        w[2] = col[2];
        w[3] = col[3];
    }
}

// Bloom test (eq 8) of one staged matcher row: lane l takes location l
// (l < 64; further locations from probes in LDS), ANDs the row bits at its
// probe positions, and the row passes if any lane's location has all of
// them.  pr0 holds lane l's first kp (padded, a multiple of 4) positions.
__device__ __forceinline__ bool bloom_row_test(const uint32_t *row, const uint4 *pr0,
                                               const uint32_t *probes, int n_loc, int kp,
                                               int lane) {
    uint32_t all = lane < n_loc ? 1u : 0u;
#pragma unroll
    for (int q = 0; q < MAX_KP / 4; ++q)
        if (q * 4 < kp) {
            const uint4 pp = pr0[q];
            all &= (row[pp.x >> 5] >> (pp.x & 31u)) & (row[pp.y >> 5] >> (pp.y & 31u)) &
                   (row[pp.z >> 5] >> (pp.z & 31u)) & (row[pp.w >> 5] >> (pp.w & 31u));
        }
    if (lane < n_loc)
        for (int q = MAX_KP; q < kp; q += 4) {   // probes past the registers
            const uint4 pp = *(const uint4 *)(probes + lane * kp + q);
            all &= (row[pp.x >> 5] >> (pp.x & 31u)) & (row[pp.y >> 5] >> (pp.y & 31u)) &
                   (row[pp.z >> 5] >> (pp.z & 31u)) & (row[pp.w >> 5] >> (pp.w & 31u));
        }
    bool any = __ballot(all & 1u) != 0ull;
    for (int lg = 64; lg < n_loc && !any; lg += 64) {   // uniform
        const int l = lg + lane;
        uint32_t a2 = l < n_loc ? 1u : 0u;
        if (l < n_loc) {
            const uint4 *pr = (const uint4 *)(probes + l * kp);
            for (int q = 0; q < kp; q += 4) {
                const uint4 pp = pr[q >> 2];
                a2 &= (row[pp.x >> 5] >> (pp.x & 31u)) & (row[pp.y >> 5] >> (pp.y & 31u)) &
                      (row[pp.z >> 5] >> (pp.z & 31u)) & (row[pp.w >> 5] >> (pp.w & 31u));
            }
        }
        any = __ballot(a2 & 1u) != 0ull;
    }
    return any;
}

// Bitonic sort of n2 (power of two) keys in LDS, descending, with payload.
__device__ void bitonic_desc(uint64_t *key, int32_t *idx, int n2) {
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n2; i += blockDim.x) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool desc = (i & size) == 0;
                    const uint64_t a = key[i], c = key[j];
                    if (desc ? (a < c) : (a > c)) {
                        key[i] = c;
                        key[j] = a;
                        const int32_t t = idx[i];
                        idx[i] = idx[j];
                        idx[j] = t;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Number of keys in key[lo .. hi) greater than x, four LDS reads in flight.
__device__ __forceinline__ int count_above(const uint64_t *key, int lo, int hi, uint64_t x) {
    int r = 0, q = lo;
    for (; q + 4 <= hi; q += 4) {
        const uint64_t a0 = key[q], a1 = key[q + 1], a2 = key[q + 2], a3 = key[q + 3];
        r += (int)(a0 > x) + (int)(a1 > x) + (int)(a2 > x) + (int)(a3 > x);
    }
    for (; q < hi; ++q) r += key[q] > x;
    return r;
}

__device__ __forceinline__ int next_pow2(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Reorder writes of output slot sl (GRACE Section 3.3, Section 5.3): a live
// slot takes the key's parent row, token, score and child node and copies
// the parent's token and block-table rows (block ids only); a dead slot is
// -1 / -inf throughout.
__device__ __forceinline__ void write_slot(const TailParams &p, int b, size_t sl, bool live,
                                           uint64_t key, int32_t child) {
    const int V = p.V, L = p.L, t = p.t;
    if (live) {
        const uint32_t f = key_flat(key);
        const int m = (int)(f / (uint32_t)V), v = (int)(f % (uint32_t)V);
        const int parent = b * p.M_in + m;
        // the parent's rows are read before any store of the slot: stores
        // count in the same counter as loads, so a store ahead of them
        // would make their wait cover its completion too
        if (p.vec_rows) {   // rows of L int32 as 16-byte pieces
            auto piece = [&](int l0) {
                int4 tk = make_int4(-1, -1, -1, -1), tb = tk;
                if (p.tokens_out && l0 < t) tk = *(const int4 *)(p.tokens_in + (size_t)parent * L + l0);
                if (p.table_out && l0 <= t) tb = *(const int4 *)(p.table_in + (size_t)parent * L + l0);
                int *tkv = (int *)&tk, *tbv = (int *)&tb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int l = l0 + e;
                    tkv[e] = l < t ? tkv[e] : (l == t ? v : -1);
                    tbv[e] = l <= t ? tbv[e] : -1;
                }
                if (p.tokens_out) *(int4 *)(p.tokens_out + sl * L + l0) = tk;
                if (p.table_out) *(int4 *)(p.table_out + sl * L + l0) = tb;
            };
            piece(0);   // the first piece outside a loop: no wait at a loop entry
            for (int l0 = 4; l0 < L; l0 += 4) piece(l0);
        } else {
            if (p.tokens_out)
                for (int l = 0; l < L; ++l)
                    p.tokens_out[sl * L + l] = l < t ? p.tokens_in[(size_t)parent * L + l] : (l == t ? v : -1);
            if (p.table_out)
                for (int l = 0; l < L; ++l)
                    p.table_out[sl * L + l] = l <= t ? p.table_in[(size_t)parent * L + l] : -1;
        }
        p.parent_out[sl] = parent;
        p.token_out[sl] = v;
        p.node_out[sl] = child;
        p.acc_out[sl] = key_score(key);
    } else {
        p.parent_out[sl] = -1;
        p.token_out[sl] = -1;
        p.node_out[sl] = -1;
        p.acc_out[sl] = -INFINITY;
        if (p.tokens_out)
            for (int l = 0; l < L; ++l) p.tokens_out[sl * L + l] = -1;
        if (p.table_out)
            for (int l = 0; l < L; ++l) p.table_out[sl * L + l] = -1;
    }
}

// ---------------------------------------------------------------------------
// Node-major pass at the step after the root.  There every live beam row of a
// request sits at a different child of the root, so the rows of all requests
// at one root child can be tested together against that node's bit-sliced
// block: the workgroups of a node run on one XCD, so the block goes through
// one L2 once instead of once per request.  One wavefront takes one
// request's row.  The row of request b at root child n is the one the
// inverse map names (recorded by the previous step's select); a row belongs
// to this pass when the map names it, its node is n and n has a block, and
// k_expand skips exactly those rows, so any map content gives the same
// result and a map from the previous step covers every row.
// ---------------------------------------------------------------------------
constexpr int NM_WAVES = EXP_WAVES;   // the pass runs in k_expand's workgroups
static_assert(NM_MAX_GX <= SEL_THREADS, "k_select takes one segment per thread with node-major parts");

__device__ __forceinline__ int nth_set_bit(uint64_t x, int n) {
    for (int i = 0; i < n; ++i) x &= x - 1;
    return __builtin_ctzll(x);
}

// eqs 5 and 8 for every child of a bit-sliced block, for one request, by one
// wavefront.  Column pos of the block is the wc words at blk + pos * wc (bit
// j of word u: child 64 u + j); the block has c children.  A column is read
// as NP = wc / PW pieces of PW words by LPC lanes (a power of two >= NP), so
// one load instruction reads CPI = 64 / LPC whole columns -- a few cache
// lines -- rather than a line per lane.  Lane (g, j) = (lane / LPC, lane %
// LPC) ANDs piece j of its slot g's attribute columns (eq 5), which the
// slots then combine; eq 8 takes the user's locations CPI at a time, lane
// (g, j) ANDing the probe columns of location g of the group, and the slots
// OR their results into the running ANY.  The groups stop as soon as every
// child that passes eq 5 has a location with all its probe bits: further
// locations cannot change the result (the OR only grows), and the Bloom rows
// of shallow nodes -- unions over many ads -- are dense enough that the
// first group usually covers every child.  Lanes j < NP of slot 0 return the
// pass bits of words PW j .. PW j + PW - 1.  ubm: the request's attribute
// word; spr: the wavefront's copy in LDS of the user's probe positions,
// location l's at spr[l * NM_KP ..] (l < n_loc <= 64; written by the
// wavefront and ordered before the call).
template <int PW>
__device__ __forceinline__ void sliced_pass(const uint64_t *blk, int wc, int c, int bl_pos,
                                            uint64_t ubm, const uint16_t *spr, int n_loc,
                                            int bloom_k, bool bloom, int lane, uint64_t out[PW]) {
    const int NP = wc / PW;
    int lg = 0;
    while ((1 << lg) < NP) ++lg;
    const int LPC = 1 << lg, CPI = 64 >> lg;
    const int g = lane >> lg, j = lane & (LPC - 1);
    const bool jv = j < NP;
    auto load = [&](int pos, uint64_t v[PW]) {
        const uint64_t *col = blk + (size_t)pos * wc + PW * j;
        if constexpr (PW == 2) {
            const uint4 u = *(const uint4 *)col;
            v[0] = (uint64_t)u.x | ((uint64_t)u.y << 32);
            v[1] = (uint64_t)u.z | ((uint64_t)u.w << 32);
        } else {
            v[0] = *col;
        }
    };
    uint64_t att[PW], acc[PW];
#pragma unroll
    for (int e = 0; e < PW; ++e) {
        att[e] = ~0ull;
        acc[e] = 0ull;
    }
    const int nub = __popcll(ubm);
    for (int u0 = 0; u0 < nub; u0 += CPI) {
        const int u = u0 + g;
        if (jv && u < nub) {
            uint64_t v[PW];
            load(bl_pos + nth_set_bit(ubm, u), v);
#pragma unroll
            for (int e = 0; e < PW; ++e) att[e] &= v[e];
        }
    }
    // the slots of a piece: lanes j, j + LPC, j + 2 LPC, ...
    for (int o = LPC; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < PW; ++e) att[e] &= __shfl_xor(att[e], o, 64);
    if (!bloom) {
#pragma unroll
        for (int e = 0; e < PW; ++e) out[e] = att[e];
        return;
    }
    // children of this lane's piece that pass eq 5 and that no location
    // has covered yet
    uint64_t need[PW];
#pragma unroll
    for (int e = 0; e < PW; ++e) {
        const int rem = c - 64 * (PW * j + e);
        const uint64_t vm = rem >= 64 ? ~0ull : (rem > 0 ? (1ull << rem) - 1ull : 0ull);
        need[e] = jv ? att[e] & vm : 0ull;
    }
    for (int l0 = 0; l0 < n_loc; l0 += CPI) {   // uniform
        uint64_t any_need = 0ull;
#pragma unroll
        for (int e = 0; e < PW; ++e) any_need |= need[e];
        if (__ballot(any_need != 0ull) == 0ull) break;
        const int l = l0 + g;
        const bool lv = jv && l < n_loc;
        uint32_t pos[NM_KP];
#pragma unroll
        for (int k = 0; k < NM_KP; ++k) pos[k] = spr[(lv ? l : 0) * NM_KP + k];
        uint64_t v[NM_KP][PW];
#pragma unroll
        for (int k = 0; k < NM_KP; ++k)   // every probe column first, then the ANDs
            if (k < bloom_k && lv) load(pos[k], v[k]);
        uint64_t a[PW];
#pragma unroll
        for (int e = 0; e < PW; ++e) a[e] = lv ? ~0ull : 0ull;
#pragma unroll
        for (int k = 0; k < NM_KP; ++k)
            if (k < bloom_k && lv)
#pragma unroll
                for (int e = 0; e < PW; ++e) a[e] &= v[k][e];
#pragma unroll
        for (int e = 0; e < PW; ++e) acc[e] |= a[e];
        for (int o = LPC; o < 64; o <<= 1)
#pragma unroll
            for (int e = 0; e < PW; ++e) acc[e] |= __shfl_xor(acc[e], o, 64);
#pragma unroll
        for (int e = 0; e < PW; ++e) need[e] &= ~acc[e];
    }
#pragma unroll
    for (int e = 0; e < PW; ++e) out[e] = att[e] & acc[e];
}

// Node-major workgroup k (at the front of k_expand's grid): request b at
// NM_WAVES consecutive root children, one wavefront per child.  The
// workgroups of one group of children, one per request, have the same k
// mod 8, so they run on one XCD, one after another, and read the children's
// blocks through one L2.  The workgroup shares the request's bound and a
// histogram of its survivors' bins, added to the request's histogram one
// atomic per bin in use (an atomic per survivor, many lanes of one
// instruction on the same bin, cost more than the whole pass).
template <bool BF16>
__device__ __forceinline__ void expand_nm(const TailParams &p, int k, uint64_t *s_dyn) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int xcd = k & 7, q = k >> 3;
    const int ng = (q / p.B) * 8 + xcd, b = q % p.B;
    if (ng * NM_WAVES >= p.n_nm) return;   // the whole workgroup
    const int ni = ng * NM_WAVES + wave, node = ni + 1;   // this wavefront's root child
    const int V = p.V, words = (V + 63) >> 6;
    uint32_t *s_h = (uint32_t *)s_dyn;                                    // survivors' bins
    float *s_ubw = (float *)(s_h + NBINS);                                // bound per wavefront
    uint32_t *s_cp = (uint32_t *)(s_ubw + 4);                             // histogram sum per wavefront
    // the row's logits, as they are in memory (bf16 bits or fp32), then
    // the pass words
    float *s_xw = s_ubw + 8 + (size_t)wave * p.nm_wave_dw;
    float *s_x = s_xw;
    uint16_t *s_xh = (uint16_t *)s_xw;
    uint64_t *s_pw = (uint64_t *)(s_xw + (BF16 ? ((V + 7) & ~7) / 2 : (V + 3) & ~3));
    auto xat = [&](int v) -> float {   // logit v of the row
        if constexpr (BF16) return bf16_to_f32(s_xh[v]);
        else return s_x[v];
    };
    uint64_t *s_tm = s_pw + ((words + 1) & ~1);                            // kept tokens (debug)
    uint16_t *s_pr = (uint16_t *)(s_tm + ((words + 1) & ~1));              // the user's probes

    // The row the map names, the node's children and block, the request's
    // attribute word and this lane's location's probes: one round of loads.
    const bool has_node = ni < p.n_nm;
    const int m = has_node ? p.inv[(size_t)b * V + ni] : -1;
    const int32_t o0 = has_node ? p.off[node] : 0, o1 = has_node ? p.off[node + 1] : 0;
    const int64_t blk = has_node && p.nslice ? p.nslice[node] : -1;
    const uint64_t ubm = p.user_bm[(size_t)b * p.w_bm];
    // lane l: location l's probe positions, into the wavefront's LDS copy
    // (below 2^16: bloom_bits <= 65536), where the block test reads them
#pragma unroll
    for (int kk = 0; kk < NM_KP; ++kk)
        s_pr[lane * NM_KP + kk] = (uint16_t)((p.w_bl && lane < p.n_loc && kk < p.bloom_k)
                                                 ? p.user_probes[((size_t)b * p.n_loc + lane) * p.bloom_k + kk] &
                                                       (uint32_t)(p.bloom_bits - 1)
                                                 : 0u);
    for (int i = tid; i < NBINS; i += EXP_THREADS) s_h[i] = 0u;
    // The row's node (whether the row is this pass's), its score and its
    // first logits need only m, so they are loaded together; a row that
    // turns out not to be the pass's drops them.
    const bool in_range = m >= 0 && m < p.M_in && blk >= 0;
    const size_t r = (size_t)b * p.M_in + (in_range ? m : 0);
    const int32_t nd = in_range ? p.node_in[r] : -1;
    const float acc = in_range ? p.acc_in[r] : 0.0f;
    const bool vec = BF16 && p.vec_logits;
    const uint4 *x8 = (const uint4 *)((const uint16_t *)p.logits + r * V);
    uint4 lgv[NM_LG];   // 8 logits per piece, NM_LG pieces per lane up front
#pragma unroll
    for (int q = 0; q < NM_LG; ++q) {
        const int cc = lane + 64 * q;
        lgv[q] = vec && in_range && cc < (V >> 3) ? x8[cc] : make_uint4(0u, 0u, 0u, 0u);
    }
    // the request's bound: the same live rows and the same max as k_select
    {
        const BoundLoads bl = bound_load(p, b);
        const float ub = bound_finish(p, b, bl);
        if (lane == 0) s_ubw[wave] = ub;
    }
    const bool active = in_range && nd == node;   // wave-uniform
    const int c = o1 - o0, wc = (c + 63) >> 6;
    float lse = 0.0f;
    uint32_t cutv = 0u;
    if (active) {
        // log-sum-exp over all V logits; the logits stay in LDS for the scores
        float mx = -INFINITY;
        if (vec) {
            auto take8 = [&](int cc, const uint4 &u) {
                *(uint4 *)(s_xh + 8 * cc) = u;
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    mx = fmaxf(mx, fmaxf(__uint_as_float(w4[h] << 16), __uint_as_float(w4[h] & 0xFFFF0000u)));
            };
#pragma unroll
            for (int q = 0; q < NM_LG; ++q)
                if (lane + 64 * q < (V >> 3)) take8(lane + 64 * q, lgv[q]);
            for (int cc = lane + 64 * NM_LG; cc < (V >> 3); cc += 64) take8(cc, x8[cc]);
        } else {
            for (int v = lane; v < V; v += 64) {
                if constexpr (BF16) {
                    const uint16_t u = ((const uint16_t *)p.logits)[r * V + v];
                    s_xh[v] = u;
                    mx = fmaxf(mx, bf16_to_f32(u));
                } else {
                    const float x = logit_at<BF16>(p.logits, r * V + v);
                    s_x[v] = x;
                    mx = fmaxf(mx, x);
                }
            }
        }
        mx = wave_max(mx);
        wave_lds_sync();
        float se = 0.0f;
        if (mx != -INFINITY)
            for (int v = lane; v < V; v += 64) se += __expf(xat(v) - mx);
        se = wave_sum(se);
        lse = mx + __logf(se);

        // eqs 5 and 8 for every child
        const uint64_t *bp = p.slice_tab + blk;
        const int bl_pos = p.w_bl ? p.bloom_bits : 0;
        // the request's cutoff counters, read now, used at the survivors
        cutv = lane < NCUT_USED ? p.cut[(size_t)b * NCUT + lane] : 0u;
        wave_lds_sync();   // the probes' LDS copy
        if ((wc & 1) == 0) {
            uint64_t pw[2];
            sliced_pass<2>(bp, wc, c, bl_pos, ubm, s_pr, p.n_loc, p.bloom_k, p.w_bl != 0, lane, pw);
            if (lane < (wc >> 1)) {
                s_pw[2 * lane] = pw[0];
                s_pw[2 * lane + 1] = pw[1];
            }
        } else {
            uint64_t pw[1];
            sliced_pass<1>(bp, wc, c, bl_pos, ubm, s_pr, p.n_loc, p.bloom_k, p.w_bl != 0, lane, pw);
            if (lane < wc) s_pw[lane] = pw[0];
        }
        if (p.mask_words)
            for (int w = lane; w < words; w += 64) s_tm[w] = 0ull;
    }
    // the wavefronts' bounds and the cleared histogram, needed from here on
    __syncthreads();
    const float U = fmaxf(fmaxf(s_ubw[0], s_ubw[1]), fmaxf(s_ubw[2], s_ubw[3]));
    if (active) {
        // Candidates past the first cutoff bin that already holds k counted
        // survivors of the request cannot be selected (the threshold bin lies
        // at or below that cutoff, and the counts only grow), so they are
        // dropped: written nowhere, counted nowhere.
        const uint64_t full = __ballot(lane < NCUT_USED && cutv >= (uint32_t)p.k_out);
        const int bmax = full ? cut_bin(__builtin_ctzll(full)) : NBINS;
        // pass 1: the kept children of each word (their mask replaces the
        // word's pass bits) and their number.  A node with all V children has
        // tokens 0 .. V - 1 in entry order (sorted and distinct), so its
        // tokens need no loads.
        const bool dense = c == V;
        uint32_t n = 0;
        for (int u0 = 0; u0 < wc; u0 += NM_SW) {   // NM_SW words: every load of the chunk in flight
            int tk[NM_SW];
            bool ok[NM_SW];
#pragma unroll
            for (int q2 = 0; q2 < NM_SW; ++q2) {
                const int u = u0 + q2, jj = 64 * u + lane;
                ok[q2] = u < wc && jj < c && ((s_pw[u < wc ? u : 0] >> lane) & 1ull);
                tk[q2] = ok[q2] ? (dense ? jj : p.tok[o0 + jj]) : 0;
            }
#pragma unroll
            for (int q2 = 0; q2 < NM_SW; ++q2) {
                if (u0 + q2 >= wc) break;   // uniform
                const float sc = ok[q2] ? acc + (xat(tk[q2]) - lse) : -INFINITY;
                if (ok[q2] && p.mask_words)
                    atomicOr((unsigned long long *)&s_tm[tk[q2] >> 6], 1ull << (tk[q2] & 63));
                const bool keep = ok[q2] && sc > -INFINITY && score_bin(sc, U) <= bmax;
                const uint64_t bal = __ballot(keep);
                if (lane == 0) s_pw[u0 + q2] = bal;
                n += (uint32_t)__popcll(bal);
            }
        }
        wave_lds_sync();
        // pass 2: the kept children reserved at the back of the segment of
        // the row's row-major workgroup (m mod gx), a multiple of 8
        const uint32_t n8 = (n + 7u) & ~7u;
        const int xs = m % p.gx;
        const uint64_t seg_cap = (uint64_t)p.seg_cap;
        uint32_t old = 0;
        if (lane == 0 && n8) old = atomicAdd(&p.segback[(size_t)b * NM_MAX_GX + xs], n8);
        old = __builtin_amdgcn_readlane(old, 0);
        const bool room = (uint64_t)old + n8 <= seg_cap;   // false only with a dirty workspace
        const size_t base = ((size_t)b * p.gx + xs) * seg_cap + (seg_cap - old - n8);
        uint32_t e = 0;   // survivors written (uniform)
        for (int u0 = 0; u0 < wc && e < n; u0 += NM_SW) {
            int tk[NM_SW], ch[NM_SW];
            bool ok[NM_SW];
#pragma unroll
            for (int q2 = 0; q2 < NM_SW; ++q2) {
                const int u = u0 + q2, jj = 64 * u + lane;
                ok[q2] = u < wc && ((s_pw[u < wc ? u : 0] >> lane) & 1ull);
                tk[q2] = ok[q2] ? (dense ? jj : p.tok[o0 + jj]) : 0;
                ch[q2] = ok[q2] ? p.child[o0 + jj] : 0;
            }
#pragma unroll
            for (int q2 = 0; q2 < NM_SW; ++q2) {
                if (u0 + q2 >= wc) break;   // uniform
                const float sc = ok[q2] ? acc + (xat(tk[q2]) - lse) : -INFINITY;
                const uint64_t bal = __ballot(ok[q2]);
                if (ok[q2] && room) {
                    const size_t idx = base + e + lanes_below(bal);
                    const int bin = score_bin(sc, U);
                    p.skey[idx] = make_key(sc, (uint32_t)(m * V + tk[q2]));
                    p.schild[idx] = ch[q2];
                    p.sbin[idx] = (uint16_t)bin;
                    atomicAdd(&s_h[bin], 1u);
                }
                e += (uint32_t)__popcll(bal);
            }
        }
        if (room)   // the reserved slots past the survivors are pads
            for (uint32_t i = e + lane; i < n8; i += 64) {
                p.skey[base + i] = 0ull;
                p.sbin[base + i] = 0xFFFFu;
            }
        if (p.mask_words) {   // debug outputs of the row
            wave_lds_sync();
            if (p.dbg_mask)
                for (int w = lane; w < words; w += 64) p.dbg_mask[r * words + w] = s_tm[w];
            if (p.dbg_scores)
                for (int v = lane; v < V; v += 64) {
                    const bool kept = (s_tm[v >> 6] >> (v & 63)) & 1ull;
                    p.dbg_scores[r * V + v] = kept ? acc + (xat(v) - lse) : -INFINITY;
                }
        }
    }
    // the workgroup's bins into the request's histogram, and its counts at
    // or below each cutoff bin into the request's counters: an inclusive
    // prefix sum over bins 0 .. 1023 (4 consecutive bins per thread), left
    // in place of those bins and read at the cutoffs
    static_assert(4 * EXP_THREADS == 1024 && NBINS >= 1024, "cutoff bins");
    __syncthreads();
    uint32_t *gh = p.hist + (size_t)b * NBINS;
    for (int i = tid; i < NBINS; i += EXP_THREADS) {
        const uint32_t cnt = s_h[i];
        if (cnt) atomicAdd(&gh[i], cnt);
    }
    uint32_t c4[4], t4 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        c4[q] = s_h[4 * tid + q];
        t4 += c4[q];
    }
    const uint32_t inc = wave_incl_sum(t4);   // inclusive prefix over the lanes
    if (lane == 63) s_cp[wave] = inc;
    __syncthreads();   // every bin read (above and by the merge), the wave totals written
    uint32_t run = inc - t4;
    for (int w = 0; w < wave; ++w) run += s_cp[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        run += c4[q];
        s_h[4 * tid + q] = run;
    }
    __syncthreads();
    if (tid < NCUT_USED) {
        const uint32_t t = s_h[cut_bin(tid)];
        if (t) atomicAdd(&p.cut[(size_t)b * NCUT + tid], t);
    }
}

// The node-major pass as its own launch: no row-major state, so it holds
// fewer registers and less LDS and more of its workgroups share a CU:
// seven wavefronts per SIMD (72 registers, about 20 KB of LDS per
// workgroup at V = 1024); at eight the spills cost more than the pass
// gains, the memory system being what then bounds it.
template <bool BF16>
__global__ __launch_bounds__(EXP_THREADS) __attribute__((amdgpu_waves_per_eu(7)))
void k_expand_nm(TailParams p) {
    extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];
    expand_nm<BF16>(p, (int)blockIdx.x, s_dyn);
}

// One workgroup = up to rows_wg beam rows of one request, taken with a stride
// of gx (row m = x + i * gx) so that the live rows,
// which sit at the front of a request after a top-k, spread over the grid.
// The CSR child entries of those rows are flattened and processed 64 at a
// time, one entry per lane: token, child, bitmask test (eq 5); then the Bloom
// test (eq 8) for the entries that passed.  WIDE (rows of >= 64 words): the
// rows of up to 64 * NQ / w_bl entries are loaded into registers in one
// round, then moved to LDS G rows at a time for the test; otherwise G rows
// are loaded straight into LDS per sub-round.
template <bool BF16, bool WIDE>
__global__ __launch_bounds__(EXP_THREADS) __attribute__((amdgpu_waves_per_eu(4)))
void k_expand(TailParams p) {
    extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];  // [mask][probes][staging]
    __shared__ uint32_t s_hist[NBINS];
    __shared__ uint64_t s_ubm[MAX_WBM];
    __shared__ int32_t s_rstart[MAX_ROWS_WG + 1];  // prefix sums of child counts
    __shared__ int32_t s_nstart[MAX_ROWS_WG + 1];  // the same over rows without a block
    __shared__ int32_t s_roff[MAX_ROWS_WG];        // first CSR entry of the row's node
    __shared__ int32_t s_rm[MAX_ROWS_WG];          // beam index m of the row
    __shared__ float s_lse[MAX_ROWS_WG];
    __shared__ float s_acc[MAX_ROWS_WG];
    __shared__ int64_t s_rblk[MAX_ROWS_WG];        // bit-sliced block of the row's node
    __shared__ uint8_t s_skip[MAX_ROWS_WG];        // the row is the node-major pass's
    __shared__ uint32_t s_nsurv;                   // survivors written to the segment
    __shared__ int32_t s_slist[MAX_ROWS_WG];       // rows with a bit-sliced block
    __shared__ int s_nsl;
    __shared__ int32_t s_sck[MAX_ROWS_WG];         // first chunk item of each listed row
    __shared__ int s_nck;                          // chunk items over all listed rows
    __shared__ float s_ub[EXP_WAVES];
    __shared__ int s_nub;
    __shared__ int32_t s_lb[2 * EXP_THREADS];      // the round's Bloom rows awaiting eq 8
                                                   //   (-1 once the test fails)
    __shared__ uint32_t s_lf[EXP_THREADS];         // k-way: the thread that listed a row
    __shared__ uint32_t s_nl;                      // entries in the list
    __shared__ uint32_t s_kn;                      // k-way: partitions listed this sub-round
    __shared__ uint8_t s_kok[EXP_THREADS];         // k-way: entry kept (a partition passed)

    // a flat grid: the node-major workgroups (p.nm_wgs, the longer ones)
    // first, then gx * B row-major workgroups (x fastest)
    const int gx = p.gx;
    if ((int)blockIdx.x < p.nm_wgs) {
        expand_nm<BF16>(p, (int)blockIdx.x, s_dyn);
        return;
    }
    const int flat = (int)blockIdx.x - p.nm_wgs;
    const int b = flat / gx, x = flat - b * gx;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nrows = x < p.M_in ? min(p.rows_wg, (p.M_in - x + gx - 1) / gx) : 0;
    const int V = p.V, words = (V + 63) >> 6;
    const int kp = (p.bloom_k + 3) & ~3;   // probes per location, padded
    const int nprobe = p.w_bl ? p.n_loc * kp : 0;
    uint64_t *s_mask = s_dyn;
    uint64_t *s_pass = s_dyn + (((size_t)p.rows_wg * p.mask_words + 1) & ~(size_t)1);
    uint16_t *s_lg = (uint16_t *)(s_pass + (((size_t)p.rows_wg * p.wmax + 1) & ~(size_t)1));
    uint32_t *s_probe = (uint32_t *)(s_lg + (p.lds_lg ? (size_t)p.rows_wg * V : 0));
    int16_t *s_ubit = (int16_t *)(s_probe + nprobe);   // positions of the user's bitmask bits
    uint32_t *s_stage = s_probe + nprobe + (p.wmax ? 32 * p.w_bm : 0) + wave * p.stage_dw;

    for (int i = tid; i < NBINS; i += EXP_THREADS) s_hist[i] = 0u;
    for (int i = tid; i < p.w_bm; i += EXP_THREADS) s_ubm[i] = p.user_bm[(size_t)b * p.w_bm + i];
    for (int i = tid; i < nprobe; i += EXP_THREADS) {
        const int l = i / kp, q = i - l * kp;
        const int qs = q < p.bloom_k ? q : 0;   // pad with the location's first probe
        s_probe[i] = p.user_probes[((size_t)b * p.n_loc + l) * p.bloom_k + qs] & (uint32_t)(p.bloom_bits - 1);
    }
    for (int i = tid; i < p.rows_wg * p.mask_words; i += EXP_THREADS) s_mask[i] = 0ull;
    if (tid == 0) {
        s_nsurv = 0u;
        s_nl = 0u;
        s_kn = 0u;
    }
    const BoundLoads bl0 = bound_load(p, b);   // reduced just before the barrier
    if (p.wmax && wave == 1) {  // list the user's attribute bits (eq 5 columns)
        const uint64_t u = lane < p.w_bm ? p.user_bm[(size_t)b * p.w_bm + lane] : 0ull;
        const int n = __popcll(u);
        int inc = n;
        inc = (int)wave_incl_sum((uint32_t)inc);   // inclusive prefix over the lanes
        uint64_t x = u;
        for (int q = inc - n; x; ++q) {
            s_ubit[q] = (int16_t)(lane * 64 + __builtin_ctzll(x));
            x &= x - 1;
        }
        if (lane == 63) s_nub = inc;
    }

    // Rows of this workgroup, their child ranges and the prefix sum of counts.
    if (wave == 0) {
        int cnt = 0;
        if (lane < nrows) {
            const int m = x + lane * gx;
            const int r = b * p.M_in + m;
            const int node = p.node_in[r];
            int off0 = 0;
            float acc = -INFINITY;
            int64_t blk = -1;
            bool skip = false;
            if (node >= 0 && node < p.num_nodes) {  // otherwise a dead row
                off0 = p.off[node];
                cnt = p.off[node + 1] - off0;
                acc = p.acc_in[r];
                if (p.nslice) blk = p.nslice[node];
                if (nm_covered(p, b, m, node, blk)) {   // tested by k_expand_nm
                    skip = true;
                    cnt = 0;
                    blk = -1;
                }
            }
            s_skip[lane] = skip;
            s_rblk[lane] = blk;
            s_roff[lane] = off0;
            s_rm[lane] = m;
            s_acc[lane] = acc;
        }
        int inc = cnt;
        inc = (int)wave_incl_sum((uint32_t)inc);   // inclusive prefix over the lanes
        if (lane < nrows) s_rstart[lane + 1] = inc;
        if (lane == 0) s_rstart[0] = 0;
        const uint64_t sl = __ballot(lane < nrows && cnt > 0 && s_rblk[lane < nrows ? lane : 0] >= 0);
        if ((sl >> lane) & 1ull) s_slist[__popcll(sl & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0) s_nsl = __popcll(sl);
        // a listed row is processed in chunks of 4 column words (4 * 64
        // children), one wavefront per chunk, so the chunks of a wide row
        // run side by side; chunk items are numbered row by row
        const int nck = ((sl >> lane) & 1ull) ? (((cnt + 63) >> 6) + 3) >> 2 : 0;
        const int inc3 = (int)wave_incl_sum((uint32_t)nck);   // inclusive prefix over the lanes
        if ((sl >> lane) & 1ull) s_sck[__popcll(sl & ((1ull << lane) - 1ull))] = inc3 - nck;
        if (lane == 63) s_nck = inc3;
        // prefix over the rows without a block: their entries go through the rounds
        int inc2 = ((sl >> lane) & 1ull) ? 0 : cnt;
        inc2 = (int)wave_incl_sum((uint32_t)inc2);   // inclusive prefix over the lanes
        if (lane < nrows) s_nstart[lane + 1] = inc2;
        if (lane == 0) s_nstart[0] = 0;
    }
    // Full-vocabulary log-sum-exp of every live row (eq 3 masks
    // log-probabilities, so the normaliser runs over all V tokens): TPR
    // threads per row, each with a running (max, sum) over its share.
    {
        const int tpr = p.tpr, sh_tpr = p.log2_tpr;
        const int i = tid >> sh_tpr, part = tid & (tpr - 1);
        float m = -INFINITY, s = 0.0f;
        // the row's node decides whether it is live; its logits are read
        // while wavefront 0 is still resolving the rows' CSR ranges
        bool has = false;
        size_t rowoff = 0;
        if (i < nrows) {
            const int r = b * p.M_in + x + i * gx;
            const int nd = p.node_in[r];
            has = nd >= 0 && nd < p.num_nodes;
            if (has && p.n_nm && nd >= 1 && nd <= p.n_nm)   // a node-major row needs no LSE here
                has = !nm_covered(p, b, x + i * gx, nd, p.nslice ? p.nslice[nd] : -1);
            rowoff = (size_t)r * V;
        }
        if (has) {
            if (BF16 && p.vec_logits) {
                // 8 logits per 16-byte load and up to 8 loads in flight per
                // thread; then one max and one rescaled sum per batch
                const uint4 *x8 = (const uint4 *)((const uint16_t *)p.logits + rowoff);
                const int nv = V >> 3;
                for (int c0 = part; c0 < nv; c0 += 8 * tpr) {
                    uint4 u[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int c = c0 + q * tpr;
                        u[q] = c < nv ? x8[c] : make_uint4(0u, 0u, 0u, 0u);
                    }
                    if (p.lds_lg)   // kept for the candidates' scores
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int c = c0 + q * tpr;
                            if (c < nv) *(uint4 *)(s_lg + (size_t)i * V + c * 8) = u[q];
                        }
                    float mx = m;
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (c0 + q * tpr < nv) {
                            const uint32_t w4[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
                            for (int h = 0; h < 4; ++h)
                                mx = fmaxf(mx, fmaxf(__uint_as_float(w4[h] << 16),
                                                     __uint_as_float(w4[h] & 0xFFFF0000u)));
                        }
                    if (mx == -INFINITY) continue;   // nothing finite yet
                    float sm = m == -INFINITY ? 0.0f : s * __expf(m - mx);
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (c0 + q * tpr < nv) {
                            const uint32_t w4[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
                            for (int h = 0; h < 4; ++h)
                                sm += __expf(__uint_as_float(w4[h] << 16) - mx) +
                                      __expf(__uint_as_float(w4[h] & 0xFFFF0000u) - mx);
                        }
                    m = mx;
                    s = sm;
                }
            } else {
                for (int v = part; v < V; v += tpr) lse_push(logit_at<BF16>(p.logits, rowoff + v), m, s);
            }
        }
        // merge the (max, sum) pairs of the row's tpr threads, butterfly
        // fashion: within 16 lanes on DPP when tpr >= 16, by permutes beyond
        auto merge = [&](float m2, float s2) {
            const float mm = fmaxf(m, m2);
            s = (m == -INFINITY ? 0.0f : s * __expf(m - mm)) + (m2 == -INFINITY ? 0.0f : s2 * __expf(m2 - mm));
            m = mm;
        };
        int o0 = 1;
        if (tpr >= 16) {   // uniform
            merge(dpp_f32<0xB1>(m), dpp_f32<0xB1>(s));     // lane ^ 1
            merge(dpp_f32<0x4E>(m), dpp_f32<0x4E>(s));     // lane ^ 2
            merge(dpp_f32<0x141>(m), dpp_f32<0x141>(s));   // mirror within 8
            merge(dpp_f32<0x140>(m), dpp_f32<0x140>(s));   // mirror within 16
            o0 = 16;
        }
        for (int o = o0; o < tpr; o <<= 1) merge(__shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
        if (i < nrows && part == 0) s_lse[i] = has ? m + __logf(s) : 0.0f;
    }
    {
        const float ub = bound_finish(p, b, bl0);
        if (lane == 0) s_ub[wave] = ub;
    }
    __syncthreads();
    const float U = fmaxf(fmaxf(s_ub[0], s_ub[1]), fmaxf(s_ub[2], s_ub[3]));
    // this workgroup's survivor segment: slots come from an LDS counter
    uint64_t *skey = p.skey + ((size_t)b * gx + x) * p.seg_cap;
    int32_t *schild = p.schild + ((size_t)b * gx + x) * p.seg_cap;
    uint16_t *sbin = p.sbin + ((size_t)b * gx + x) * p.seg_cap;
    const int G = p.G, wq = p.w_bl, sh_wq = p.log2_wq;
    const int row_dw = 2 * wq + 1;   // staged row stride in dwords (odd: spreads banks)

    // A candidate that passed CD + TM with a finite score: its bin in the
    // workgroup histogram and its (key, child) in the segment.  Called by
    // whole wavefronts.
    auto emit = [&](bool sel, float score, uint32_t f, int32_t ch) {
        const int bin = score_bin(score, U);
        if (sel) atomicAdd(&s_hist[bin], 1u);
        const uint64_t bal = __ballot(sel);
        if (bal) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_nsurv, (uint32_t)__popcll(bal));
            base = __builtin_amdgcn_readlane(base, 0);
            if (sel) {
                const uint32_t idx = base + lanes_below(bal);
                if (idx < (uint32_t)p.seg_cap) {
                    skey[idx] = make_key(score, f);
                    schild[idx] = ch;
                    sbin[idx] = (uint16_t)bin;
                }
            }
        }
    };
    auto mark = [&](int i, int v) {   // debug mask bit of row i, token v
        atomicOr((unsigned long long *)&s_mask[i * p.mask_words + (v >> 6)], 1ull << (v & 63));
    };

    // lane l's location l: its probe positions, kept in registers
    uint4 pr0[MAX_KP / 4];
#pragma unroll
    for (int q = 0; q < MAX_KP / 4; ++q) {
        pr0[q] = make_uint4(0u, 0u, 0u, 0u);
        if (q * 4 < kp && lane < p.n_loc && p.w_bl) pr0[q] = ((const uint4 *)(s_probe + lane * kp))[q];
    }


    // logit of token v of the workgroup's row i (beam m): from LDS when the
    // log-sum-exp pass kept the rows there, else from memory
    auto row_logit = [&](int i, int m, int v) -> float {
        if (p.lds_lg) return bf16_to_f32(s_lg[(size_t)i * V + v]);
        return logit_at<BF16>(p.logits, (size_t)(b * p.M_in + m) * V + v);
    };

    // eqs 5 and 8 for every child of a node with a bit-sliced block, one
    // wavefront per chunk of 4 column words (256 children) of a row.  Eq 5:
    // AND of the columns of the user's attribute bits.  Eq 8: lane l ANDs
    // the columns of location l's probe positions (bit j set = child j has
    // all of them), then the lanes OR (ANY location).
    if (p.wmax) {
        const int nub = s_nub, nsl = s_nsl;
        const int bl_pos = p.w_bl ? p.bloom_bits : 0;
        const int ub0 = nub ? s_ubit[lane < nub ? lane : 0] : 0;   // lane's user bit
        const int nitems = s_nck;
        for (int it = wave; it < nitems; it += EXP_WAVES) {
            int li = 0;   // the listed row of chunk item it, and its chunk ck
            while (li + 1 < nsl && s_sck[li + 1] <= it) ++li;
            const int ck = it - s_sck[li];
            const int i = s_slist[li];
            const int64_t blk = s_rblk[i];
            const int c = s_rstart[i + 1] - s_rstart[i];
            const int wc = (c + 63) >> 6;
            const uint64_t *tab = p.slice_tab + blk;
            if (wc == 1) {
                // one word per column (fewer than 65 children): every load
                // first, then one AND and one OR reduction
                uint64_t bm = lane < nub ? tab[bl_pos + ub0] : ~0ull;
                for (int qg = 64; qg < nub; qg += 64)   // user bits past 64
                    if (qg + lane < nub) bm &= tab[bl_pos + s_ubit[qg + lane]];
                uint64_t acc = 0ull;
                if (p.w_bl) {
                    uint64_t a = ~0ull;
#pragma unroll
                    for (int qq = 0; qq < MAX_KP / 4; ++qq)
                        if (qq * 4 < kp)
                            a &= tab[pr0[qq].x] & tab[pr0[qq].y] & tab[pr0[qq].z] & tab[pr0[qq].w];
                    if (lane < p.n_loc)
                        for (int q = MAX_KP; q < kp; q += 4) {   // probes past the registers
                            const uint4 pp = *(const uint4 *)(s_probe + lane * kp + q);
                            a &= tab[pp.x] & tab[pp.y] & tab[pp.z] & tab[pp.w];
                        }
                    acc = lane < p.n_loc ? a : 0ull;
                    for (int lg = 64; lg < p.n_loc; lg += 64) {   // locations past 64
                        const int l = lg + lane;
                        if (l < p.n_loc) {
                            uint64_t a2 = ~0ull;
                            const uint4 *pr = (const uint4 *)(s_probe + l * kp);
                            for (int q = 0; q < kp; q += 4) {
                                const uint4 pp = pr[q >> 2];
                                a2 &= tab[pp.x] & tab[pp.y] & tab[pp.z] & tab[pp.w];
                            }
                            acc |= a2;
                        }
                    }
                }
                uint64_t pass = wave_and64(bm);
                if (p.w_bl) pass &= wave_or64(acc);
                if (lane == 0) s_pass[(size_t)i * p.wmax] = pass;
            } else {
            const bool even = (wc & 1) == 0;
            for (int w0 = 4 * ck; w0 < min(wc, 4 * ck + 4); w0 += 4) {   // this chunk
                const int n = min(4, wc - w0);
                // every column load of the row first, the reductions after
                uint64_t bm[4];
                col4(tab + (size_t)(bl_pos + ub0) * wc + w0, even, bm);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (lane >= nub) bm[u] = ~0ull;
                for (int qg = 64; qg < nub; qg += 64) {   // user bits past 64
                    const int q = qg + lane;
                    if (q < nub) {
                        uint64_t cw[4];
                        col4(tab + (size_t)(bl_pos + s_ubit[q]) * wc + w0, even, cw);
#pragma unroll
                        for (int u = 0; u < 4; ++u) bm[u] &= cw[u];
                    }
                }
                uint64_t acc[4] = {0ull, 0ull, 0ull, 0ull};
                if (p.w_bl) {
                    uint64_t a[4] = {~0ull, ~0ull, ~0ull, ~0ull};
#pragma unroll
                    for (int qq = 0; qq < MAX_KP / 4; ++qq)
                        if (qq * 4 < kp) {
                            // the pads of the last group (copies of the
                            // location's first probe) are not loaded again
                            const int bk = p.bloom_k - qq * 4;   // real probes in this group
                            uint64_t c0[4], c1[4], c2[4], c3[4];
                            col4(tab + (size_t)pr0[qq].x * wc + w0, even, c0);
                            if (bk > 1) col4(tab + (size_t)pr0[qq].y * wc + w0, even, c1);
                            if (bk > 2) col4(tab + (size_t)pr0[qq].z * wc + w0, even, c2);
                            if (bk > 3) col4(tab + (size_t)pr0[qq].w * wc + w0, even, c3);
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                uint64_t x = c0[u];
                                if (bk > 1) x &= c1[u];
                                if (bk > 2) x &= c2[u];
                                if (bk > 3) x &= c3[u];
                                a[u] &= x;
                            }
                        }
                    if (lane < p.n_loc)
                        for (int q = MAX_KP; q < kp; q += 4) {   // probes past the registers
                            const uint4 pp = *(const uint4 *)(s_probe + lane * kp + q);
                            const uint32_t pos[4] = {pp.x, pp.y, pp.z, pp.w};
                            for (int t4 = 0; t4 < 4; ++t4) {
                                uint64_t cw[4];
                                col4(tab + (size_t)pos[t4] * wc + w0, even, cw);
#pragma unroll
                                for (int u = 0; u < 4; ++u) a[u] &= cw[u];
                            }
                        }
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[u] = lane < p.n_loc ? a[u] : 0ull;
                    for (int lg = 64; lg < p.n_loc; lg += 64) {   // locations past 64
                        const int l = lg + lane;
                        if (l < p.n_loc) {
                            uint64_t a2[4] = {~0ull, ~0ull, ~0ull, ~0ull};
                            const uint4 *pr = (const uint4 *)(s_probe + l * kp);
                            for (int q = 0; q < kp; q += 4) {
                                const uint4 pp = pr[q >> 2];
                                const uint32_t pos[4] = {pp.x, pp.y, pp.z, pp.w};
                                for (int t4 = 0; t4 < 4; ++t4) {
                                    uint64_t cw[4];
                                    col4(tab + (size_t)pos[t4] * wc + w0, even, cw);
#pragma unroll
                                    for (int u = 0; u < 4; ++u) a2[u] &= cw[u];
                                }
                            }
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[u] |= a2[u];
                        }
                    }
                }
                uint64_t pass[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (u < n) {   // uniform
                        pass[u] = wave_and64(bm[u]);
                        if (p.w_bl) pass[u] &= wave_or64(acc[u]);
                    }
                if (lane < n) {
                    uint64_t x = pass[0];
#pragma unroll
                    for (int u = 1; u < 4; ++u)
                        if (lane == u) x = pass[u];
                    s_pass[(size_t)i * p.wmax + w0 + lane] = x;
                }
            }
            }
            wave_lds_sync();
            // The row's candidates: the children whose pass bit is set, 64
            // per chunk and up to 4 chunks of loads in flight.
            const int off0 = s_roff[i], m = s_rm[i];
            const float acc = s_acc[i], lse = s_lse[i];
            const uint64_t *pw = s_pass + (size_t)i * p.wmax;
            for (int u0 = 4 * ck; u0 < min(wc, 4 * ck + 4); u0 += 4) {   // this chunk
                int tk[4], ch[4];
                bool okc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int u = u0 + q, jj = u * 64 + lane;
                    okc[q] = u < wc && jj < c && ((pw[u < wc ? u : 0] >> lane) & 1ull);
                    tk[q] = 0;
                    ch[q] = 0;
                    if (okc[q]) {
                        tk[q] = p.tok[off0 + jj];
                        ch[q] = p.child[off0 + jj];
                    }
                }
                float xv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[q] = okc[q] ? row_logit(i, m, tk[q]) : 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (u0 + q >= wc) break;   // uniform
                    const float sc = okc[q] ? acc + (xv[q] - lse) : -INFINITY;
                    if (okc[q] && p.mask_words) mark(i, tk[q]);
                    emit(okc[q] && sc > -INFINITY, sc, (uint32_t)(m * V + tk[q]), ch[q]);
                }
            }
        }
    }
    __syncthreads();

    // eq 8 for a list of n_bl Bloom row ids lb[0 .. n_bl): ANY user location
    // whose probe bits are all set in the row.  The wavefronts share the
    // list; a row that fails becomes -1.  Called by the whole workgroup.
    auto bloom_list = [&](int32_t *lb, int n_bl) {
        if (WIDE) {
            // CH rows per wavefront batch, loaded into registers in one round
            // (register q holds 8-byte word ((q * 64) mod w_bl) + lane of row
            // (q * 64) / w_bl), then moved to LDS G rows at a time.
            const int CH = (64 * NQ) >> sh_wq;
            for (int g0 = wave * CH; g0 < n_bl; g0 += EXP_WAVES * CH) {
                const int nq = min(CH, n_bl - g0);
                const int myrow = lane < nq ? lb[g0 + lane] : -1;
                uint2 r[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    // the row id is uniform: a scalar buffer descriptor per row,
                    // empty (loads return 0, no memory access) past the list
                    const int g = (q << 6) >> sh_wq;
                    const int rid = __builtin_amdgcn_readlane(myrow, g);
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(p.bl_tab + (size_t)(rid < 0 ? 0 : rid) * wq), (short)0,
                        rid < 0 ? 0 : wq * 8, BUF_DWORD3);
                    const auto u = __builtin_amdgcn_raw_buffer_load_b64(
                        rs, lane * 8, ((q << 6) & (wq - 1)) * 8, 0);
                    r[q] = make_uint2(u[0], u[1]);
                }
                uint64_t pm = 0ull;
                for (int s0 = 0; s0 < nq; s0 += G) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const int g = (q << 6) >> sh_wq;
                        if (g >= s0 && g < s0 + G) {
                            uint32_t *dst = s_stage + 2 * lane +
                                            ((g - s0) * row_dw + 2 * ((q << 6) & (wq - 1)));
                            dst[0] = r[q].x;
                            dst[1] = r[q].y;
                        }
                    }
                    wave_lds_sync();
                    for (int g = 0; g < G && s0 + g < nq; ++g)
                        if (bloom_row_test(s_stage + g * row_dw, pr0, s_probe, p.n_loc, kp, lane))
                            pm |= 1ull << (s0 + g);
                    wave_lds_sync();
                }
                if (lane < nq && !((pm >> lane) & 1ull)) lb[g0 + lane] = -1;
            }
        } else {
            // G rows per wavefront batch, loaded straight into LDS
            for (int g0 = wave * G; g0 < n_bl; g0 += EXP_WAVES * G) {
                const int nq = min(G, n_bl - g0);
                const int nld = nq << sh_wq;   // 8-byte words to stage
                for (int base = 0; base < nld; base += 4 * 64) {
                    uint2 u[4];
                    int dsto[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int idx = base + q * 64 + lane;
                        dsto[q] = -1;
                        if (idx < nld) {
                            const int g = idx >> sh_wq, cw = idx & (wq - 1);
                            u[q] = *(const uint2 *)(p.bl_tab + (size_t)lb[g0 + g] * wq + cw);
                            dsto[q] = g * row_dw + 2 * cw;
                        }
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (dsto[q] >= 0) {
                            s_stage[dsto[q]] = u[q].x;
                            s_stage[dsto[q] + 1] = u[q].y;
                        }
                }
                wave_lds_sync();
                uint64_t pm = 0ull;
                for (int g = 0; g < nq; ++g)
                    if (bloom_row_test(s_stage + g * row_dw, pr0, s_probe, p.n_loc, kp, lane))
                        pm |= 1ull << g;
                wave_lds_sync();
                if (lane < nq && !((pm >> lane) & 1ull)) lb[g0 + lane] = -1;
            }
        }
    };

    // The entries of rows without a bit-sliced block, one per thread per
    // round (two with one-union matchers), the round count the same for
    // every thread.
    const int n_ent = s_nstart[nrows];
    // entry e's row, CSR position, token, child and matcher ids / rows, in
    // one round of loads
    struct Ent {
        bool valid;
        int i, j, v, bmi, bli, child, m;
        uint64_t bw0, bw1;
    };
    auto load_entry = [&](int e) {
        Ent t{};
        t.valid = e < n_ent;
        t.bli = -1;
        if (!t.valid) return t;
        int lo = 0, hi = nrows;   // the largest i with s_nstart[i] <= e
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_nstart[mid] <= e) lo = mid;
            else hi = mid;
        }
        t.i = lo;
        t.j = s_roff[lo] + (e - s_nstart[lo]);
        t.v = p.tok[t.j];
        t.child = p.child[t.j];
        if (p.ent_bm) {
            t.bw0 = p.ent_bm[(size_t)t.j * p.w_bm];
            if (p.w_bm > 1) t.bw1 = p.ent_bm[(size_t)t.j * p.w_bm + 1];
        } else {
            t.bmi = p.bmi[t.j];
        }
        if (wq) t.bli = p.bli[t.j];
        t.m = s_rm[lo];
        return t;
    };
    // eq 5: every user attribute bit present in the entry's row
    auto bitmask_ok = [&](const Ent &t) {
        if (p.ent_bm)
            return (t.bw0 & s_ubm[0]) == s_ubm[0] && (p.w_bm < 2 || (t.bw1 & s_ubm[1]) == s_ubm[1]);
        const uint64_t *bmr = p.bm_tab + (size_t)t.bmi * p.w_bm;
        for (int w = 0; w < p.w_bm; ++w)
            if ((bmr[w] & s_ubm[w]) != s_ubm[w]) return false;
        return true;
    };
    auto logit_of = [&](const Ent &t) {
        return t.valid ? row_logit(t.i, t.m, t.v) : 0.0f;
    };

    if (p.kw_off) {
        // k-way partitioned matchers: an entry is kept when one of its
        // partitions passes eq 5 and, with a Bloom matcher, eq 8.
        // Sub-rounds: every entry still undecided offers its next partition
        // that passes eq 5; the offered Bloom rows are tested together by
        // all wavefronts.
        for (int c0 = 0; c0 < n_ent; c0 += EXP_THREADS) {
            const Ent t = load_entry(c0 + tid);
            const float xk = logit_of(t);
            int cur = t.valid ? p.kw_off[t.j] : 0;
            const int q1 = t.valid ? p.kw_off[t.j + 1] : 0;
            auto bm_pass = [&](int q) {
                const uint64_t *r = p.bm_tab + (size_t)p.kw_bmi[q] * p.w_bm;
                for (int w = 0; w < p.w_bm; ++w)
                    if ((r[w] & s_ubm[w]) != s_ubm[w]) return false;
                return true;
            };
            bool kept = false;
            if (!wq) {
                while (!kept && cur < q1) kept = bm_pass(cur++);
            } else {
                s_kok[tid] = 0;
                int32_t *lb = s_lb;
                for (;;) {   // the same number of sub-rounds for every thread
                    int32_t blr = -1;
                    while (!kept && cur < q1) {
                        const int q = cur++;
                        if (bm_pass(q)) {
                            blr = p.kw_bli[q];
                            break;
                        }
                    }
                    const uint64_t dm = __ballot(blr >= 0);
                    if (dm) {
                        uint32_t base = 0;
                        if (lane == 0) base = atomicAdd(&s_kn, (uint32_t)__popcll(dm));
                        base = __builtin_amdgcn_readlane(base, 0);
                        if (blr >= 0) {
                            const uint32_t qi = base + lanes_below(dm);
                            lb[qi] = blr;
                            s_lf[qi] = (uint32_t)tid;
                        }
                    }
                    __syncthreads();
                    const int n_k = (int)s_kn;
                    if (n_k == 0) break;   // uniform
                    bloom_list(lb, n_k);
                    __syncthreads();
                    if (tid < n_k && lb[tid] >= 0) s_kok[s_lf[tid]] = 1;
                    __syncthreads();
                    kept = kept || s_kok[tid] != 0;
                    if (tid == 0) s_kn = 0u;
                    __syncthreads();
                }
            }
            const float sk = kept ? s_acc[t.i] + (xk - s_lse[t.i]) : -INFINITY;
            if (kept && p.mask_words) mark(t.i, t.v);
            emit(kept && sk > -INFINITY, sk, (uint32_t)(t.m * V + t.v), t.child);
        }
    } else {
        // One-union matchers: two entries per thread per round, both
        // entries' loads issued before either is used.  Entries that pass
        // eq 5 put their Bloom row on the round's list (up to 2 *
        // EXP_THREADS), which all wavefronts test together (eq 8); the
        // owner then emits its entries that passed.  The scores are not
        // needed before that, so the logit gathers overlap the Bloom loads.
        int32_t *Lb = s_lb;
        for (int c0 = 0; c0 < n_ent; c0 += 2 * EXP_THREADS) {
            const Ent t0 = load_entry(c0 + tid), t1 = load_entry(c0 + EXP_THREADS + tid);
            const float x0 = logit_of(t0), x1 = logit_of(t1);
            const Ent *ts[2] = {&t0, &t1};
            const float xs[2] = {x0, x1};
            int qs[2] = {-1, -1};   // the entry's place in the list
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const Ent &t = *ts[u];
                const bool ok = t.valid && bitmask_ok(t);
                if (!wq) {   // bitmask-only matcher: decided now
                    const float score = ok ? s_acc[t.i] + (xs[u] - s_lse[t.i]) : -INFINITY;
                    if (ok && p.mask_words) mark(t.i, t.v);
                    emit(ok && score > -INFINITY, score, (uint32_t)(t.m * V + t.v), t.child);
                    continue;
                }
                const uint64_t dm = __ballot(ok);
                if (dm) {
                    uint32_t base = 0;
                    if (lane == 0) base = atomicAdd(&s_nl, (uint32_t)__popcll(dm));
                    base = __builtin_amdgcn_readlane(base, 0);
                    if (ok) {
                        qs[u] = (int)(base + lanes_below(dm));
                        Lb[qs[u]] = t.bli;
                    }
                }
            }
            if (!wq) continue;   // bitmask-only matcher: no Bloom test, no list
            __syncthreads();
            const int n_bl = (int)s_nl;
            if (n_bl) {   // uniform
                // eq 8 for the round's list (a failed entry's row id becomes -1)
                bloom_list(Lb, n_bl);
                __syncthreads();
                if (tid == 0) s_nl = 0u;   // every thread has read the count
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const Ent &t = *ts[u];
                const bool kept = qs[u] >= 0 && Lb[qs[u]] >= 0;
                const float score = kept ? s_acc[t.i] + (xs[u] - s_lse[t.i]) : -INFINITY;
                if (kept && p.mask_words) mark(t.i, t.v);
                emit(kept && score > -INFINITY, score, (uint32_t)(t.m * V + t.v), t.child);
            }
            __syncthreads();   // the list is rewritten by the next round
        }
    }

    if (p.mask_words) {  // debug outputs: kept tokens and their scores, per row
        __syncthreads();
        for (int i = wave; i < nrows; i += EXP_WAVES) {
            if (s_skip[i]) continue;   // written by the node-major pass
            const size_t r = (size_t)b * p.M_in + s_rm[i];
            const uint64_t *mk = s_mask + i * p.mask_words;
            if (p.dbg_mask)
                for (int w = lane; w < words; w += 64) p.dbg_mask[r * words + w] = mk[w];
            if (p.dbg_scores)
                for (int v = lane; v < V; v += 64) {
                    const bool kept = (mk[v >> 6] >> (v & 63)) & 1ull;
                    p.dbg_scores[r * V + v] =
                        kept ? s_acc[i] + (logit_at<BF16>(p.logits, r * V + v) - s_lse[i]) : -INFINITY;
                }
        }
    }

    // Merge this workgroup's histogram into the request's and publish the
    // segment's count; k_select reads both after the kernel boundary, so no
    // device-scope fence is needed here.
    __syncthreads();
    {   // pad the segment to a multiple of 8 (seg_cap is one)
        const uint32_t n = min(s_nsurv, (uint32_t)p.seg_cap);
        const uint32_t n8 = (n + 7u) & ~7u;
        if ((uint32_t)tid < n8 - n) {
            skey[n + tid] = 0ull;
            sbin[n + tid] = 0xFFFFu;
        }
        if (tid == 0) p.segcnt[(size_t)b * gx + x] = n8;
    }
    uint32_t *gh = p.hist + (size_t)b * NBINS;
    for (int i = tid; i < NBINS; i += EXP_THREADS) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

__global__ __launch_bounds__(SEL_THREADS) void k_select(TailParams p) {
    __shared__ uint32_t s_seg[NBINS];     // bin starts, then (after the scatter) bin ends
    __shared__ uint64_t s_key[MAX_K];     // winners, grouped by bin
    __shared__ int32_t s_src[MAX_K];      // their survivor index
    __shared__ uint64_t s_bkey[BND_CAP];  // members of the threshold bin
    __shared__ int32_t s_bsrc[BND_CAP];
    __shared__ uint32_t s_wsum[SEL_THREADS / 64];
    __shared__ uint32_t s_cnt[256];
    __shared__ uint32_t s_segpre[MAX_GX + 1];  // prefix sums of the segments' survivors
    __shared__ uint32_t s_wsum2[SEL_THREADS / 64];
    __shared__ int s_thr, s_below, s_nbnd, s_ncol, s_digit, s_rem;
    __shared__ uint32_t s_cand[CAND_CAP];     // survivors in bins up to the threshold bin
    __shared__ uint32_t s_ncand, s_ncl;

    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ float s_ub[SEL_THREADS / 64];
    const int k = p.k_out;
    // survivors of request b: segment x holds segcnt[b, x] keys at
    // keys + x * seg_cap; a survivor is named by its offset in the request
    const int gx = p.gx;
    const uint64_t seg_cap = (uint64_t)p.seg_cap;
    const uint64_t *keys = p.skey + (size_t)b * gx * seg_cap;
    uint32_t *gh = p.hist + (size_t)b * NBINS;
    // The segment counts and this thread's histogram bins are loaded before
    // the bound's rows, so the three reads share one round trip.  The
    // survivors are listed as sub-segments: with a node-major pass, segment
    // x has a front part (its workgroup's survivors) and a back part (the
    // node-major survivors of its rows, at the segment's end), thread tid
    // taking both of segment tid; otherwise thread tid takes segments 2 tid
    // and 2 tid + 1.  Every sub-segment holds a multiple of 8 entries.
    const uint32_t *cnt = p.segcnt + (size_t)b * gx;
    const bool two = p.n_nm != 0;                               // then gx <= NM_MAX_GX
    const int nsub = two ? 2 * gx : gx;                         // <= 2 * SEL_THREADS
    uint32_t c0, c1;
    if (two) {
        c0 = tid < gx ? min(cnt[tid], (uint32_t)seg_cap) & ~7u : 0u;
        c1 = tid < gx ? p.segback[(size_t)b * NM_MAX_GX + tid] & ~7u : 0u;
        if (c1 > (uint32_t)seg_cap - c0) c1 = 0u;   // only with a dirty workspace
        if (tid < gx) p.segback[(size_t)b * NM_MAX_GX + tid] = 0u;   // zero for the next call
    } else {
        c0 = 2 * tid < gx ? cnt[2 * tid] : 0u;       // gx <= 2 * SEL_THREADS
        c1 = 2 * tid + 1 < gx ? cnt[2 * tid + 1] : 0u;
    }
    constexpr int PER = NBINS / SEL_THREADS;
    uint32_t c[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) c[i] = gh[tid * PER + i];
    {
        const float ub = bound_part(p, b);
        if (lane == 0) s_ub[wave] = ub;
    }
    {   // exclusive prefix of the segment counts
        uint32_t sinc = c0 + c1;
        sinc = wave_incl_sum(sinc);   // inclusive prefix over the lanes
        if (lane == 63) s_wsum2[wave] = sinc;
        __syncthreads();
        uint32_t spre = 0;
        for (int w = 0; w < wave; ++w) spre += s_wsum2[w];
        const uint32_t ex = spre + sinc - c0 - c1;
        // thread tid writes entries 2 tid and 2 tid + 1; entry nsub (the
        // total) lies past the last thread's pair when nsub = 2 * SEL_THREADS
        if (2 * tid <= nsub) s_segpre[2 * tid] = ex;
        if (2 * tid + 1 <= nsub) s_segpre[2 * tid + 1] = ex + c0;
        if (nsub == 2 * SEL_THREADS && tid == SEL_THREADS - 1) s_segpre[nsub] = ex + c0 + c1;
    }
    float U = s_ub[0];
    for (int w = 1; w < SEL_THREADS / 64; ++w) U = fmaxf(U, s_ub[w]);

    // 1. Exclusive prefix of the score histogram (read above, zeroed here
    //    for the next call: the workspace stays zero-filled between calls);
    //    the threshold bin is the one that holds the k-th best survivor.
    uint32_t part = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) part += c[i];
#pragma unroll
    for (int i = 0; i < PER; ++i) gh[tid * PER + i] = 0u;
    if (tid < NCUT) p.cut[(size_t)b * NCUT + tid] = 0u;   // zero for the next call too
    for (int i = tid; i < MAX_K; i += SEL_THREADS) s_key[i] = 0ull;
    uint32_t inc = part;
    inc = wave_incl_sum(inc);   // inclusive prefix over the lanes
    if (lane == 63) s_wsum[wave] = inc;
    if (tid == 0) {
        s_thr = NBINS;
        s_nbnd = 0;
        s_ncol = 0;
        s_ncand = 0xFFFFFFFFu;   // every survivor (no threshold bin)
    }
    __syncthreads();
    uint32_t pre = 0, total = 0;
    for (int w = 0; w < SEL_THREADS / 64; ++w) {
        const uint32_t x = s_wsum[w];
        pre += w < wave ? x : 0u;
        total += x;
    }
    uint32_t cum = pre + inc - part;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        s_seg[tid * PER + i] = cum;
        if (total > (uint32_t)k && cum < (uint32_t)k && (uint32_t)k <= cum + c[i]) {
            s_thr = tid * PER + i;
            s_below = (int)cum;
            s_ncand = cum + c[i];   // survivors in bins up to and including this one
        }
        cum += c[i];
    }
    if (tid == 0 && total <= (uint32_t)k) s_below = (int)total;
    if (tid == 0) s_ncl = 0u;
    __syncthreads();
    const int thr = s_thr, below = s_below;
    uint32_t n_surv = 0;   // the total of the segment counts
    for (int w = 0; w < SEL_THREADS / 64; ++w) n_surv += s_wsum2[w];
    // the sub-segment holding the f-th survivor (sub-segments concatenated)
    auto sub_of = [&](uint32_t f) -> int {
        int lo = 0, hi = nsub;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_segpre[mid] <= f) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    // offset in the request's keys of the f-th survivor, in sub-segment lo
    // (survivors s_segpre[lo] .. s_segpre[lo + 1] - 1)
    auto off_in = [&](int lo, uint32_t f) -> uint32_t {
        if (!two) return (uint32_t)(lo * seg_cap) + (f - s_segpre[lo]);
        const uint32_t seg = (uint32_t)lo >> 1;
        if (!(lo & 1)) return (uint32_t)(seg * seg_cap) + (f - s_segpre[lo]);
        return (uint32_t)((seg + 1) * seg_cap) - (s_segpre[lo + 1] - f);   // a back part
    };
    auto surv = [&](uint32_t f) -> uint32_t { return off_in(sub_of(f), f); };

    // 2. Survivors of bins below the threshold go to their bin's slots;
    //    members of the threshold bin are buffered.  Zero keys are the
    //    segments' pads.
    auto take = [&](uint64_t key, uint32_t src) {
        if (key == 0ull) return;
        const int bin = score_bin(key_score(key), U);
        if (bin < thr) {
            const uint32_t pos = atomicAdd(&s_seg[bin], 1u);
            if (pos < (uint32_t)MAX_K) {
                s_key[pos] = key;
                s_src[pos] = (int32_t)src;
            }
        } else if (bin == thr) {
            const int pos = atomicAdd(&s_nbnd, 1);
            if (pos < BND_CAP) {
                s_bkey[pos] = key;
                s_bsrc[pos] = (int32_t)src;
            }
        }
    };
    if (n_surv >= BIN_SCAN_MIN && s_ncand <= CAND_CAP) {
        // Many survivors: their bins are read 8 at a time (16 bytes, 4 groups
        // in flight per thread); the positions of bins at or below the
        // threshold bin go to an LDS list, whose keys are then fetched all at
        // once.  Pads carry bin 0xFFFF.
        const uint16_t *bins = p.sbin + (size_t)b * gx * seg_cap;
        const uint32_t n_oct = n_surv >> 3;
        for (uint32_t o0 = 0; o0 < n_oct; o0 += 4 * SEL_THREADS) {
            // wavefront w takes 256 consecutive groups, lane l groups l,
            // l + 64, l + 128, l + 192 of them (each load instruction reads
            // 1 KB in one piece); a lane searches for its sub-segment once
            // and again only when a later group lies past it
            uint32_t src[4];
            uint4 bv[4];
            int lo = -1;
            uint32_t end = 0;   // first survivor past sub-segment lo
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t oo = o0 + (uint32_t)wave * 256u + (uint32_t)u * 64u + (uint32_t)lane;
                src[u] = 0xFFFFFFFFu;
                if (oo < n_oct) {
                    const uint32_t f = 8 * oo;
                    if (lo < 0 || f >= end) {
                        lo = sub_of(f);
                        end = s_segpre[lo + 1];
                    }
                    src[u] = off_in(lo, f);
                }
                bv[u] = src[u] != 0xFFFFFFFFu ? *(const uint4 *)(bins + src[u])
                                              : make_uint4(~0u, ~0u, ~0u, ~0u);
            }
            // bit 8u + e: survivor src[u] + e is a candidate; one LDS atomic
            // per wavefront reserves the wavefront's list positions.  Few
            // groups hold a candidate: the smallest of a group's 8 bins
            // (packed 16-bit minima) decides whether its bits are looked at.
            uint32_t msk = 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t m2 = pk_min_u16(pk_min_u16(bv[u].x, bv[u].y), pk_min_u16(bv[u].z, bv[u].w));
                const uint32_t mn = min(m2 & 0xFFFFu, m2 >> 16);
                if (src[u] != 0xFFFFFFFFu && mn <= (uint32_t)thr) {
                    const uint32_t wv[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int bn = (int)((wv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                        if (bn <= thr) msk |= 1u << (8 * u + e);
                    }
                }
            }
            const uint32_t nmine = (uint32_t)__popc(msk);
            uint32_t inc = nmine;
            inc = wave_incl_sum(inc);   // inclusive prefix over the lanes
            uint32_t base = 0;
            if (lane == 63 && inc) base = atomicAdd(&s_ncl, inc);
            base = __builtin_amdgcn_readlane(base, 63);
            uint32_t ci = base + inc - nmine;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t mm = (msk >> (8 * u)) & 0xFFu;
                while (mm) {
                    const int e = __ffs(mm) - 1;
                    mm &= mm - 1u;
                    if (ci < CAND_CAP) s_cand[ci] = src[u] + e;
                    ++ci;
                }
            }
        }
        __syncthreads();
        const uint32_t nc = min(s_ncl, (uint32_t)CAND_CAP);
        for (uint32_t c0 = 0; c0 < nc; c0 += 4 * SEL_THREADS) {
            uint32_t src[4];
            uint64_t kk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t ci = c0 + u * SEL_THREADS + tid;
                src[u] = ci < nc ? s_cand[ci] : 0xFFFFFFFFu;
                kk[u] = ci < nc ? keys[src[u]] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (src[u] != 0xFFFFFFFFu) take(kk[u], src[u]);
        }
    } else {
        // Pairs are read coalesced (consecutive threads take consecutive
        // pairs), 8 pairs in flight per thread.
        const uint32_t n_pairs = n_surv >> 1;
        for (uint32_t p0 = 0; p0 < n_pairs; p0 += 8 * SEL_THREADS) {
            // every pair's offset first, then every load (a pair past the
            // end reads the first pair again and is dropped), so no load
            // waits behind another's search
            uint32_t src[8];
            uint4 kv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t pp = p0 + u * SEL_THREADS + tid;
                src[u] = pp < n_pairs ? surv(2 * pp) : 0xFFFFFFFFu;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                kv[u] = *(const uint4 *)(keys + (src[u] != 0xFFFFFFFFu ? src[u] : 0u));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (src[u] == 0xFFFFFFFFu) continue;
                take((uint64_t)kv[u].x | ((uint64_t)kv[u].y << 32), src[u]);
                take((uint64_t)kv[u].z | ((uint64_t)kv[u].w << 32), src[u] + 1);
            }
        }
    }
    __syncthreads();

    // 3. The best k - below members of the threshold bin fill slots below..k-1.
    int n_sel = below;
    if (thr < NBINS) {
        const int need = k - below;
        int nb = s_nbnd;
        if (nb > BND_CAP) {
            // Too many to buffer: MSB-first radix select of the need-th best
            // key of the bin over global memory, then collect the winners.
            uint64_t prefix = 0, pmask = 0;
            int rem = need;
            for (int shift = 56; shift >= 0; shift -= 8) {
                for (int i = tid; i < 256; i += SEL_THREADS) s_cnt[i] = 0u;
                __syncthreads();
                for (uint32_t f = tid; f < n_surv; f += SEL_THREADS) {
                    const uint64_t key = keys[surv(f)];
                    if (key && score_bin(key_score(key), U) == thr && (key & pmask) == prefix)
                        atomicAdd(&s_cnt[(key >> shift) & 255u], 1u);
                }
                __syncthreads();
                if (tid == 0) {
                    uint32_t acc = 0;
                    for (int d = 255; d >= 0; --d) {
                        if (acc + s_cnt[d] >= (uint32_t)rem) {
                            s_digit = d;
                            s_rem = rem - (int)acc;
                            break;
                        }
                        acc += s_cnt[d];
                    }
                }
                __syncthreads();
                prefix |= (uint64_t)s_digit << shift;
                pmask |= 0xFFull << shift;
                rem = s_rem;
                __syncthreads();
            }
            for (uint32_t f = tid; f < n_surv; f += SEL_THREADS) {
                const uint32_t i = surv(f);
                const uint64_t key = keys[i];
                if (key && score_bin(key_score(key), U) == thr && key >= prefix) {
                    const int pos = atomicAdd(&s_ncol, 1);
                    if (pos < BND_CAP) {
                        s_bkey[pos] = key;
                        s_bsrc[pos] = (int32_t)i;
                    }
                }
            }
            __syncthreads();
            nb = min(s_ncol, need);
        }
        if (nb <= 256) {
            // rank by counting: keys are distinct (the flat index is part of it)
            for (int q = tid; q < nb; q += SEL_THREADS) {
                const uint64_t kq = s_bkey[q];
                const int r = count_above(s_bkey, 0, nb, kq);
                if (r < need) {
                    s_key[below + r] = kq;
                    s_src[below + r] = s_bsrc[q];
                }
            }
        } else {
            const int n2 = next_pow2(nb);
            for (int i = nb + tid; i < n2; i += SEL_THREADS) {
                s_bkey[i] = 0ull;
                s_bsrc[i] = -1;
            }
            __syncthreads();
            bitonic_desc(s_bkey, s_bsrc, n2);
            for (int i = tid; i < need; i += SEL_THREADS) {
                s_key[below + i] = s_bkey[i];
                s_src[below + i] = s_bsrc[i];
            }
        }
        n_sel = k;
    }
    __syncthreads();

    // 4. Output.  A winner of a bin below the threshold takes slot
    //    (start of its bin) + (number of better keys in its bin); the
    //    threshold-bin winners are already in order.  Slots past n_sel are dead.
    const int V = p.V;
    for (int pos = tid; pos < k; pos += SEL_THREADS) {
        const uint64_t keyp = pos < n_sel ? s_key[pos] : 0ull;
        const uint32_t fp = key_flat(keyp);
        const uint32_t srcp = (uint32_t)s_src[pos];
        // a zero key or an out-of-range survivor (only with a workspace that
        // was not zero-filled) gives a dead slot instead of a wild read
        const bool live = keyp != 0ull && fp < (uint32_t)p.M_in * (uint32_t)V &&
                          srcp < (uint32_t)(gx * seg_cap);
        int slot = pos;
        if (live && pos < below) {
            const int bin = score_bin(key_score(keyp), U);
            const int end = (int)s_seg[bin], start = bin ? (int)s_seg[bin - 1] : 0;
            slot = start + count_above(s_key, start, end, keyp);
        }
        // the child id is read unconditionally (a dead slot reads the first
        // survivor's), so it goes out with the parent's rows
        const int32_t ch = p.schild[(size_t)b * gx * seg_cap + (live ? srcp : 0u)];
        write_slot(p, b, (size_t)b * k + slot, live, keyp, live ? ch : -1);
        // the next step's node-major pass finds the row at each root child
        if (p.map_write && live && ch >= 1 && ch <= p.n_root) p.inv[(size_t)b * p.V + ch - 1] = slot;
    }
}

// ---------------------------------------------------------------------------
// The whole tail in one launch when every request enters with one beam row
// (the root step: M_0 = 1).  A row has at most V <= 1024 children, so one
// 1024-thread workgroup per request holds all of its candidates: the row's
// log-sum-exp over its V logits, eqs 5 and 8 for every child (the bit-sliced
// block through one wavefront, as in the node-major pass, or a plain test
// per child when the node has no block), the candidates placed in order in
// LDS (score descending, then token ascending, as the histogram select
// orders them: a histogram of score bins below the row's own score, its
// prefix sums, then a rank by counting inside each bin) and the reorder
// writes -- no global histogram, no segments and no second launch.  The same
// masks, scores and selection as k_expand + k_select.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(SEL_THREADS) void k_root(TailParams p) {
    __shared__ uint64_t s_key[SEL_THREADS];
    __shared__ int32_t s_ch[SEL_THREADS];
    __shared__ float s_x[SEL_THREADS];          // the row's logits (V <= 1024)
    __shared__ uint16_t s_pr[64 * NM_KP];       // the user's probe positions (block test)
    __shared__ uint64_t s_pw[SEL_THREADS / 64];  // pass words of a bit-sliced block
    __shared__ uint64_t s_tm[SEL_THREADS / 64];  // kept tokens (debug outputs)
    __shared__ float s_red[SEL_THREADS / 64];
    __shared__ uint32_t s_bin[NBINS];            // bin counts, then bin starts, then ends
    __shared__ uint32_t s_wsum[SEL_THREADS / 64];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int V = p.V, k = p.k_out, words = (V + 63) >> 6;
    const size_t r = (size_t)b;   // one row per request
    const int node = p.node_in[r];
    const bool live = node >= 0 && node < p.num_nodes;
    int32_t o0 = 0, c = 0;
    int64_t blk = -1;
    if (live) {
        o0 = p.off[node];
        c = p.off[node + 1] - o0;
        if (p.nslice) blk = p.nslice[node];
    }
    const float acc = live ? p.acc_in[r] : 0.0f;
    const uint64_t ubm = p.user_bm[(size_t)b * p.w_bm];   // one attribute word
    // thread v: logit v; thread j: child entry j (both loaded up front)
    const float x = live && tid < V ? logit_at<BF16>(p.logits, r * V + tid) : -INFINITY;
    const int32_t tk = tid < c ? (int32_t)p.tok[o0 + tid] : 0;
    const int32_t chv = tid < c ? p.child[o0 + tid] : -1;
    if (tid < V) s_x[tid] = x;
    if (tid < words) s_tm[tid] = 0ull;
    for (int i = tid; i < NBINS; i += SEL_THREADS) s_bin[i] = 0u;

    // eqs 5 and 8 for every child of a bit-sliced block: wavefront 0
    if (live && blk >= 0 && c > 0 && wave == 0) {
#pragma unroll
        for (int kk = 0; kk < NM_KP; ++kk)
            s_pr[lane * NM_KP + kk] = (uint16_t)((p.w_bl && lane < p.n_loc && kk < p.bloom_k)
                                                     ? p.user_probes[((size_t)b * p.n_loc + lane) * p.bloom_k + kk] &
                                                           (uint32_t)(p.bloom_bits - 1)
                                                     : 0u);
        wave_lds_sync();
        const int wc = (c + 63) >> 6;
        const uint64_t *bp = p.slice_tab + blk;
        const int bl_pos = p.w_bl ? p.bloom_bits : 0;
        if ((wc & 1) == 0) {
            uint64_t pw[2];
            sliced_pass<2>(bp, wc, c, bl_pos, ubm, s_pr, p.n_loc, p.bloom_k, p.w_bl != 0, lane, pw);
            if (lane < (wc >> 1)) {
                s_pw[2 * lane] = pw[0];
                s_pw[2 * lane + 1] = pw[1];
            }
        } else {
            uint64_t pw[1];
            sliced_pass<1>(bp, wc, c, bl_pos, ubm, s_pr, p.n_loc, p.bloom_k, p.w_bl != 0, lane, pw);
            if (lane < wc) s_pw[lane] = pw[0];
        }
    }
    // the row's log-sum-exp over all V logits
    float mx = wave_max(x);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    mx = s_red[0];
    for (int w = 1; w < SEL_THREADS / 64; ++w) mx = fmaxf(mx, s_red[w]);
    float se = wave_sum(tid < V && mx != -INFINITY ? __expf(x - mx) : 0.0f);
    __syncthreads();   // every wavefront has read the maxima
    if (lane == 0) s_red[wave] = se;
    __syncthreads();
    se = 0.0f;
    for (int w = 0; w < SEL_THREADS / 64; ++w) se += s_red[w];
    const float lse = mx + __logf(se);

    // child tid: kept (CD + GTM) and its key
    bool kept = false;
    if (tid < c) {
        if (blk >= 0) {
            kept = (s_pw[tid >> 6] >> (tid & 63)) & 1ull;
        } else {   // no block: the child's own rows (eq 5, then eq 8)
            const int64_t e = (int64_t)o0 + tid;
            const uint64_t row_bm = p.ent_bm ? p.ent_bm[e] : p.bm_tab[p.bmi[e]];
            kept = (row_bm & ubm) == ubm;
            if (kept && p.w_bl) {
                const uint64_t *row = p.bl_tab + (size_t)p.bli[e] * p.w_bl;
                bool any = false;
                for (int l = 0; l < p.n_loc && !any; ++l) {
                    bool all = true;
                    for (int q = 0; q < p.bloom_k && all; ++q) {
                        const uint32_t pos = p.user_probes[((size_t)b * p.n_loc + l) * p.bloom_k + q] &
                                             (uint32_t)(p.bloom_bits - 1);
                        all = (row[pos >> 6] >> (pos & 63)) & 1ull;
                    }
                    any = all;
                }
                kept = any;
            }
        }
    }
    const float sc = kept ? acc + (s_x[tk] - lse) : -INFINITY;
    if (kept && p.mask_words) atomicOr((unsigned long long *)&s_tm[tk >> 6], 1ull << (tk & 63));
    const uint64_t key = kept && sc > -INFINITY ? make_key(sc, (uint32_t)tk) : 0ull;   // flat index = token
    // the candidate's bin below the row's own score (every candidate's
    // score is at most it), counted in LDS
    const int bin = key ? score_bin(sc, acc) : 0;
    if (key) atomicAdd(&s_bin[bin], 1u);
    __syncthreads();
    if (p.mask_words) {   // debug outputs of the row
        if (p.dbg_mask)
            for (int w = tid; w < words; w += SEL_THREADS) p.dbg_mask[r * words + w] = s_tm[w];
        if (p.dbg_scores && tid < V) {
            const bool kv = (s_tm[tid >> 6] >> (tid & 63)) & 1ull;
            p.dbg_scores[r * V + tid] = kv ? acc + (x - lse) : -INFINITY;
        }
    }
    // exclusive prefix of the bins (thread tid: bins 2 tid and 2 tid + 1)
    static_assert(NBINS == 2 * SEL_THREADS, "two bins per thread");
    const uint32_t b0 = s_bin[2 * tid], b1 = s_bin[2 * tid + 1];
    const uint32_t inc = wave_incl_sum(b0 + b1);   // inclusive prefix over the lanes
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    uint32_t pre = 0, n = 0;
    for (int w = 0; w < SEL_THREADS / 64; ++w) {
        pre += w < wave ? s_wsum[w] : 0u;
        n += s_wsum[w];
    }
    pre += inc - b0 - b1;
    s_bin[2 * tid] = pre;             // bin starts: each thread writes its own two bins
    s_bin[2 * tid + 1] = pre + b0;
    __syncthreads();
    // each candidate into its bin's run (the bins' starts become their ends),
    // then its rank inside the run by counting
    if (key) {
        const uint32_t pos = atomicAdd(&s_bin[bin], 1u);
        s_key[pos] = key;
    }
    __syncthreads();
    int slot = -1;
    if (key) {
        const int end = (int)s_bin[bin], start = bin ? (int)s_bin[bin - 1] : 0;
        slot = start + count_above(s_key, start, end, key);
    }
    __syncthreads();   // every rank is counted before the keys move
    if (key) {
        s_key[slot] = key;   // slots 0 .. n - 1, in order
        s_ch[slot] = chv;
    }
    __syncthreads();

    // slot i: the i-th best candidate, dead past the last one
    for (int i = tid; i < k; i += SEL_THREADS) {
        const bool lv = (uint32_t)i < n;
        const uint64_t ki = lv ? s_key[i] : 0ull;
        const int32_t ch = lv ? s_ch[i] : -1;
        write_slot(p, b, (size_t)b * k + i, lv, ki, ch);
        // the next step's node-major pass finds the row at each root child
        if (p.map_write && lv && ch >= 1 && ch <= p.n_root) p.inv[(size_t)b * V + ch - 1] = i;
    }
}

}  // namespace

namespace {

TailParams tail_params(const TrieDev &tr, const gr_tail_args &a, size_t *shm_out) {
    TailParams p{};
    p.off = tr.node_offsets;
    p.child = tr.child_nodes;
    p.tok = tr.tokens;
    p.bmi = tr.bitmask_index;
    p.bli = tr.bloom_index;
    p.bm_tab = tr.bitmask_table;
    p.bl_tab = tr.bloom_table;
    p.nslice = tr.node_slice;
    p.slice_tab = tr.slice_table;
    p.w_bm = tr.w_bm;
    p.w_bl = tr.w_bl;
    p.bloom_k = tr.bloom_k;
    p.bloom_bits = tr.bloom_bits;
    p.num_nodes = tr.num_nodes;
    p.B = a.B;
    p.M_in = a.M_in;
    p.V = a.V;
    p.k_out = a.k_out;
    p.t = a.t;
    p.L = a.L;
    p.n_loc = tr.w_bl ? a.n_loc : 0;
    p.user_bm = a.user_bm;
    p.user_probes = a.user_probes;
    p.logits = a.logits;
    p.node_in = a.node_in;
    p.acc_in = a.acc_in;
    p.tokens_in = a.tokens_in;
    p.table_in = a.table_in;
    p.parent_out = a.parent_out;
    p.token_out = a.token_out;
    p.node_out = a.node_out;
    p.acc_out = a.acc_out;
    p.tokens_out = a.tokens_out;
    p.table_out = a.table_out;
    p.dbg_mask = a.dbg_mask;
    p.dbg_scores = a.dbg_scores;
    const TailWsLayout ly = tail_ws_layout(a.B, a.M_in, a.V);
    char *ws = (char *)a.ws;
    p.segcnt = (uint32_t *)(ws + ly.segcnt);
    p.hist = (uint32_t *)(ws + ly.hist);
    p.skey = (uint64_t *)(ws + ly.skey);
    p.schild = (int32_t *)(ws + ly.schild);
    p.sbin = (uint16_t *)(ws + ly.sbin);
    p.seg_cap = ly.shape.seg_cap;
    p.gx = ly.shape.gx;

    p.rows_wg = ly.shape.rows_wg;
    const int gx = ly.shape.gx;
    int log2_wq = 0;
    while ((1 << log2_wq) < tr.w_bl) ++log2_wq;
    p.log2_wq = log2_wq;
    const int row_bytes = (2 * tr.w_bl + 1) * 4;
    int G = 64;
    while (G > 1 && G * row_bytes > STAGE_BYTES) G >>= 1;
    p.G = G;
    p.stage_dw = tr.w_bl ? G * (2 * tr.w_bl + 1) : 0;
    p.mask_words = (a.dbg_mask || a.dbg_scores) ? (a.V + 63) / 64 : 0;
    p.wmax = tr.node_slice ? (a.V + 63) / 64 : 0;
    p.vec_logits = a.dtype == GR_BF16 && (a.V & 7) == 0 && ((uintptr_t)a.logits & 15) == 0;
    p.ent_bm = tr.entry_bitmask;
    p.kw_off = tr.kway_offsets;
    p.kw_bmi = tr.kway_bmi;
    p.kw_bli = tr.kway_bli;
    auto al16 = [](const void *x) { return ((uintptr_t)x & 15) == 0; };
    p.vec_rows = (a.L & 3) == 0 && al16(a.tokens_in) && al16(a.tokens_out) && al16(a.table_in) &&
                 al16(a.table_out);
    const int nprobe = tr.w_bl ? p.n_loc * ((tr.bloom_k + 3) & ~3) : 0;
    p.lds_lg = p.vec_logits && (size_t)p.rows_wg * a.V * 2 <= (size_t)LG_BYTES;
    // Node-major pass at the step after the root (rows at root children).
    // It pays when a column of a node's block spans whole cache lines and
    // the blocks are large (V >= 512: 1 MB per node at V = 1024, 8192-bit
    // Bloom; stress workload t = 1: 1337 -> 751 us) and when the step's rows
    // cover most root children; at V = 256 (32-byte columns) it measured
    // even with the row-major pass, which is kept there.
    p.inv = (int32_t *)(ws + ly.inv);
    p.segback = (uint32_t *)(ws + ly.segback);
    p.cut = (uint32_t *)(ws + ly.cut);
    p.n_root = tr.n_root;
    const bool nm_ok = tr.n_root > 0 && tr.node_slice && !tr.kway_offsets && tr.w_bm == 1 &&
                       (!tr.w_bl || (p.n_loc <= 64 && tr.bloom_k <= NM_KP)) && a.V >= 512;
    p.n_nm = (nm_ok && a.t == 1 && gx <= NM_MAX_GX && 2 * (int64_t)a.M_in >= tr.n_root)
                 ? tr.n_root : 0;
    p.map_write = nm_ok && a.t == 0;
    {   // per node-major wavefront: its row's logits, pass words and kept
        // tokens; workgroups: 8 * ceil(groups / 8) * B (see expand_nm)
        const int words = (a.V + 63) / 64;
        // the row's logits as stored (bf16 or fp32), then the pass words and
        // kept tokens
        const int xdw = a.dtype == GR_BF16 ? ((a.V + 7) & ~7) / 2 : (a.V + 3) & ~3;
        p.nm_wave_dw = xdw + 4 * ((words + 1) & ~1) + 32 * NM_KP;
        const int ngroups = (p.n_nm + NM_WAVES - 1) / NM_WAVES;
        p.nm_wgs = p.n_nm ? 8 * ((ngroups + 7) / 8) * a.B : 0;
    }
    const size_t shm = sizeof(uint64_t) * (((size_t)p.rows_wg * p.mask_words + 1) & ~(size_t)1) +
                       sizeof(uint64_t) * (((size_t)p.rows_wg * p.wmax + 1) & ~(size_t)1) +
                       (p.lds_lg ? sizeof(uint16_t) * (size_t)p.rows_wg * a.V : 0) +
                       sizeof(uint32_t) * ((size_t)nprobe + (p.wmax ? 32 * (size_t)tr.w_bm : 0) +
                                           (size_t)EXP_WAVES * p.stage_dw);

    int tpr = 64;
    while (tpr > 1 && tpr * p.rows_wg > EXP_THREADS) tpr >>= 1;
    p.tpr = tpr;
    int log2_tpr = 0;
    while ((1 << log2_tpr) < tpr) ++log2_tpr;
    p.log2_tpr = log2_tpr;

    (void)gx;
    *shm_out = shm;
    return p;
}

}  // namespace

hipError_t launch_constrain(const TrieDev &tr, const gr_tail_args &a, hipStream_t s) {
    size_t shm = 0;
    TailParams p = tail_params(tr, a, &shm);
    if (p.n_nm) {   // the node-major pass first, as its own launch
        // LDS: the histogram, the bounds, the wavefronts' histogram sums,
        // then the wavefronts' areas
        const size_t shm_nm = sizeof(uint32_t) * ((size_t)NBINS + 8 + (size_t)NM_WAVES * p.nm_wave_dw);
        if (a.dtype == GR_BF16) k_expand_nm<true><<<p.nm_wgs, EXP_THREADS, shm_nm, s>>>(p);
        else k_expand_nm<false><<<p.nm_wgs, EXP_THREADS, shm_nm, s>>>(p);
        p.nm_wgs = 0;   // k_expand: row-major workgroups only (n_nm still names the pass's rows)
    }
    const dim3 g1((unsigned)p.gx * (unsigned)a.B);
    const bool wide = tr.w_bl >= 64;
    if (a.dtype == GR_BF16) {
        if (wide) k_expand<true, true><<<g1, EXP_THREADS, shm, s>>>(p);
        else k_expand<true, false><<<g1, EXP_THREADS, shm, s>>>(p);
    } else {
        if (wide) k_expand<false, true><<<g1, EXP_THREADS, shm, s>>>(p);
        else k_expand<false, false><<<g1, EXP_THREADS, shm, s>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_topk_reorder(const TrieDev &tr, const gr_tail_args &a, hipStream_t s) {
    size_t shm = 0;
    const TailParams p = tail_params(tr, a, &shm);
    k_select<<<a.B, SEL_THREADS, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_tail(const TrieDev &tr, const gr_tail_args &a, hipStream_t s) {
    // one row per request: the whole tail in one workgroup per request
    // (one attribute word, the node-major pass's probe registers)
    const bool one = a.M_in == 1 && a.V <= SEL_THREADS && a.k_out <= SEL_THREADS &&
                     !tr.kway_offsets && tr.w_bm == 1 &&
                     (!tr.w_bl || (a.n_loc <= 64 && tr.bloom_k <= NM_KP));
    if (one) {
        size_t shm = 0;
        const TailParams p = tail_params(tr, a, &shm);
        if (a.dtype == GR_BF16) k_root<true><<<a.B, SEL_THREADS, 0, s>>>(p);
        else k_root<false><<<a.B, SEL_THREADS, 0, s>>>(p);
        return hipGetLastError();
    }
    hipError_t e = launch_constrain(tr, a, s);
    if (e == hipSuccess) e = launch_topk_reorder(tr, a, s);
    return e;
}

// ---------------------------------------------------------------------------
// Library-held tail scratch for callers that cannot allocate: one file-scope
// device array per GPU (each device that loads the library holds its own copy
// until the process ends).  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, once per device, and only that
// pointer is used.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[TAIL_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEV = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEV];   // device address of `scratch`, per device

__global__ __launch_bounds__(256) void k_clear_u32x4(uint4 *p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t tail_scratch(void **out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr || ((uintptr_t)ptr & 255)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_clear_hist(void *ws, int B, hipStream_t s) {
    // the histograms sit at offset 0 of the tail workspace layout, the
    // segments' back counts right after the histogram region
    const TailWsLayout ly = tail_ws_layout(B, 1, 1);
    const size_t n = (size_t)B * NBINS * sizeof(uint32_t) / sizeof(uint4);
    k_clear_u32x4<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((uint4 *)ws, n);
    const size_t n2 = (size_t)B * NM_MAX_GX * sizeof(uint32_t) / sizeof(uint4);
    k_clear_u32x4<<<(unsigned)((n2 + 255) / 256), 256, 0, s>>>(
        (uint4 *)((char *)ws + ly.segback), n2);
    const size_t n3 = (size_t)B * NCUT * sizeof(uint32_t) / sizeof(uint4);
    k_clear_u32x4<<<(unsigned)((n3 + 255) / 256), 256, 0, s>>>(
        (uint4 *)((char *)ws + ly.cut), n3);
    return hipGetLastError();
}

}  // namespace gr
