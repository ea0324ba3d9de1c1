// CD + GTM constrain, full-vocabulary log-softmax, score accumulation,
// per-request top-k and beam reorder on gfx950.
//
// GRACE Section 3.1 (decode loop), Section 3.3 (beam top-k, dynamic widths,
// paged beam rearrangement), Section 4.1 eqs 1-3 (CD, TM, -inf masking),
// Section 4.2 eq 5 (packed bitmask test), Section 4.3 eq 8 (Bloom test, ANY
// of the user's locations), Section 4.4 / Appendix A (CSR Lookup over a
// node's child entries with deduplicated matcher rows).
//
// Three launches on one stream:
//   k_tail_prep  one workgroup per request: clears the request's score
//                histogram and counters and takes U_b = the best live parent
//                score (every candidate score is <= U_b since log-probs <= 0).
//   k_expand     wavefront per beam row: log-softmax over all V logits (row
//                staged in LDS), child-entry lanes run the bitmask test then
//                the Bloom probes with early exits, survivors are compacted
//                per request (one atomic per wavefront and 64 entries) and
//                binned into a 4096-bin histogram of U_b - score; the last
//                workgroup of a request finds the bin holding the k-th best.
//   k_select     one workgroup per request: bins above the threshold bin are
//                in, the threshold bin is resolved exactly (LDS bitonic sort,
//                or an MSB radix select over global memory when it is large),
//                the k winners are sorted by (score desc, flat index asc) and
//                the reorder writes parent / token / child node / score and
//                the token and block-table rows of the new beams.
#include "gr_device.h"
#include "gr_internal.h"

namespace gr {
namespace {

constexpr int EXP_WAVES = 4;
constexpr int EXP_THREADS = 64 * EXP_WAVES;
constexpr int EXP_ROWS = 16;          // beam rows per expand workgroup
constexpr int SEL_THREADS = 1024;
constexpr int BND_CAP = 4096;         // threshold-bin entries resolved in LDS

struct TailParams {
    const int32_t *off;
    const int32_t *child;
    const int16_t *tok;
    const int32_t *bmi;
    const int32_t *bli;
    const uint64_t *bm_tab;
    const uint64_t *bl_tab;
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
    float *ubound;
    uint32_t *ctr;   // per request: [0] survivors, [1] finished workgroups,
                     // [2] threshold bin, [3] survivors in better bins
    uint32_t *hist;
    uint64_t *skey;
    int32_t *schild;
    int64_t cap;
};

// Bin of a candidate score below the request bound U (monotone
// non-increasing in the score: a better score never lands in a later bin).
__device__ __forceinline__ int score_bin(float s, float U) {
    float d = (U - s) * BIN_SCALE;
    if (!(d > 0.0f)) return 0;
    return d >= (float)(NBINS - 1) ? NBINS - 1 : (int)d;
}

// 64-bit selection key: higher = better; score first, then lower flat index.
__device__ __forceinline__ uint64_t make_key(float s, uint32_t f) {
    return ((uint64_t)f32_ord(s) << 32) | (uint64_t)(0xFFFFFFFFu - f);
}
__device__ __forceinline__ float key_score(uint64_t k) { return f32_unord((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_flat(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

__global__ __launch_bounds__(256) void k_tail_prep(TailParams p) {
    const int b = blockIdx.x, tid = threadIdx.x;
    uint32_t *h = p.hist + (size_t)b * NBINS;
    for (int i = tid; i < NBINS; i += 256) h[i] = 0u;
    if (tid < 4) p.ctr[b * 4 + tid] = 0u;
    float mx = -INFINITY;
    for (int m = tid; m < p.M_in; m += 256) {
        const int r = b * p.M_in + m;
        if (p.node_in[r] >= 0) mx = fmaxf(mx, p.acc_in[r]);
    }
    mx = wave_max(mx);
    __shared__ float s_m[4];
    if ((tid & 63) == 0) s_m[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) p.ubound[b] = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
}

template <bool BF16>
__global__ __launch_bounds__(EXP_THREADS) void k_expand(TailParams p) {
    extern __shared__ float s_x[];                 // [EXP_WAVES][V] logits of the row
    __shared__ uint32_t s_hist[NBINS];
    __shared__ uint64_t s_ubm[MAX_WBM];
    __shared__ uint32_t s_probe[MAX_PROBES];
    __shared__ uint64_t s_mask[EXP_WAVES][MAX_V / 64];
    __shared__ int s_last;
    __shared__ uint32_t s_scan[EXP_THREADS];

    const int b = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m0 = blockIdx.x * EXP_ROWS;
    const int m1 = min(p.M_in, m0 + EXP_ROWS);
    const int V = p.V, words = (V + 63) >> 6;
    const int nprobe = p.w_bl ? p.n_loc * p.bloom_k : 0;
    for (int i = tid; i < NBINS; i += EXP_THREADS) s_hist[i] = 0u;
    for (int i = tid; i < p.w_bm; i += EXP_THREADS) s_ubm[i] = p.user_bm[(size_t)b * p.w_bm + i];
    for (int i = tid; i < nprobe; i += EXP_THREADS)
        s_probe[i] = p.user_probes[(size_t)b * nprobe + i] & (uint32_t)(p.bloom_bits - 1);
    const float U = p.ubound[b];
    __syncthreads();

    float *sx = s_x + wave * V;
    uint64_t *smask = s_mask[wave];
    const uint64_t lanemask_lt = (1ull << lane) - 1ull;
    uint64_t *skey = p.skey + (size_t)b * p.cap;
    int32_t *schild = p.schild + (size_t)b * p.cap;

    for (int m = m0 + wave; m < m1; m += EXP_WAVES) {
        const int r = b * p.M_in + m;
        int node = p.node_in[r];
        if (node >= p.num_nodes) node = -1;   // not a node of this trie: dead
        const size_t rowoff = (size_t)r * V;
        // Full-vocabulary log-sum-exp (the mask is applied after, eq 3).
        float mx = -INFINITY;
        if (BF16) {
            const uint16_t *x = (const uint16_t *)p.logits + rowoff;
            for (int v = lane; v < V; v += 64) {
                float xv = bf16_to_f32(x[v]);
                sx[v] = xv;
                mx = fmaxf(mx, xv);
            }
        } else {
            const float *x = (const float *)p.logits + rowoff;
            for (int v = lane; v < V; v += 64) {
                float xv = x[v];
                sx[v] = xv;
                mx = fmaxf(mx, xv);
            }
        }
        for (int w = lane; w < words; w += 64) smask[w] = 0ull;
        mx = wave_max(mx);
        wave_lds_sync();
        float se = 0.0f;
        for (int v = lane; v < V; v += 64) se += __expf(sx[v] - mx);
        se = wave_sum(se);
        const float lse = mx + __logf(se);
        const float acc = node >= 0 ? p.acc_in[r] : -INFINITY;

        if (node >= 0) {
            const int j0 = p.off[node], j1 = p.off[node + 1];
            for (int jb = j0; jb < j1; jb += 64) {
                const int j = jb + lane;
                bool pass = false;
                uint64_t key = 0;
                int child = 0;
                if (j < j1) {
                    const int v = p.tok[j];
                    // eq 5: every user attribute bit present in the node row
                    const uint64_t *bmr = p.bm_tab + (size_t)p.bmi[j] * p.w_bm;
                    pass = true;
                    for (int w = 0; w < p.w_bm; ++w) {
                        const uint64_t u = s_ubm[w];
                        if ((bmr[w] & u) != u) { pass = false; break; }
                    }
                    // eq 8: ANY user location whose probe bits are all set
                    if (pass && p.w_bl) {
                        const uint32_t *blr = (const uint32_t *)(p.bl_tab + (size_t)p.bli[j] * p.w_bl);
                        bool any = false;
                        for (int l = 0; l < p.n_loc && !any; ++l) {
                            const uint32_t *pr = s_probe + l * p.bloom_k;
                            bool all = true;
                            for (int i = 0; i < p.bloom_k; ++i) {
                                const uint32_t pos = pr[i];
                                if (!((blr[pos >> 5] >> (pos & 31u)) & 1u)) { all = false; break; }
                            }
                            any = all;
                        }
                        pass = any;
                    }
                    if (pass) {
                        const float s = acc + (sx[v] - lse);
                        child = p.child[j];
                        atomicOr((unsigned long long *)&smask[v >> 6], 1ull << (v & 63));
                        atomicAdd(&s_hist[score_bin(s, U)], 1u);
                        key = make_key(s, (uint32_t)(m * V + v));
                    }
                }
                const uint64_t bal = __ballot(pass);
                if (bal) {
                    uint32_t base = 0;
                    if (lane == 0) base = atomicAdd(&p.ctr[b * 4 + 0], (uint32_t)__popcll(bal));
                    base = __shfl(base, 0, 64);
                    if (pass) {
                        const uint32_t idx = base + (uint32_t)__popcll(bal & lanemask_lt);
                        skey[idx] = key;
                        schild[idx] = child;
                    }
                }
            }
        }
        wave_lds_sync();
        if (p.dbg_mask)
            for (int w = lane; w < words; w += 64) p.dbg_mask[(size_t)r * words + w] = smask[w];
        if (p.dbg_scores)
            for (int v = lane; v < V; v += 64) {
                const bool kept = (smask[v >> 6] >> (v & 63)) & 1ull;
                p.dbg_scores[rowoff + v] = kept ? acc + (sx[v] - lse) : -INFINITY;
            }
        wave_lds_sync();
    }

    // Merge this workgroup's histogram into the request's.
    __syncthreads();
    uint32_t *gh = p.hist + (size_t)b * NBINS;
    for (int i = tid; i < NBINS; i += EXP_THREADS) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&p.ctr[b * 4 + 1], 1u) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Last workgroup of request b: threshold bin of the k_out-th best score.
    constexpr int PER = NBINS / EXP_THREADS;
    uint32_t c[PER];
    uint32_t part = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = __hip_atomic_load(&gh[tid * PER + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        part += c[i];
    }
    s_scan[tid] = part;
    __syncthreads();
    for (int o = 1; o < EXP_THREADS; o <<= 1) {
        const uint32_t v = tid >= o ? s_scan[tid - o] : 0u;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const uint32_t total = s_scan[EXP_THREADS - 1];
    const uint32_t excl = s_scan[tid] - part;
    const uint32_t k = (uint32_t)p.k_out;
    if (total <= k) {
        if (tid == 0) {
            p.ctr[b * 4 + 2] = NBINS;
            p.ctr[b * 4 + 3] = total;
        }
    } else if (excl < k && k <= excl + part) {
        uint32_t cum = excl;
        for (int i = 0; i < PER; ++i) {
            if (cum + c[i] >= k) {
                p.ctr[b * 4 + 2] = (uint32_t)(tid * PER + i);
                p.ctr[b * 4 + 3] = cum;
                break;
            }
            cum += c[i];
        }
    }
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

__device__ __forceinline__ int next_pow2(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

__global__ __launch_bounds__(SEL_THREADS) void k_select(TailParams p) {
    __shared__ uint64_t s_key[MAX_K];
    __shared__ int32_t s_idx[MAX_K];
    __shared__ uint64_t s_bkey[BND_CAP];
    __shared__ int32_t s_bidx[BND_CAP];
    __shared__ uint32_t s_cnt[256];
    __shared__ int s_nsel, s_nbnd, s_digit, s_rem;

    const int b = blockIdx.x, tid = threadIdx.x;
    const uint32_t N = p.ctr[b * 4 + 0];
    const uint32_t thr = p.ctr[b * 4 + 2];
    const float U = p.ubound[b];
    const int k = p.k_out;
    const uint64_t *keys = p.skey + (size_t)b * p.cap;
    if (tid == 0) {
        s_nsel = 0;
        s_nbnd = 0;
    }
    __syncthreads();
    for (uint32_t i = tid; i < N; i += SEL_THREADS) {
        const uint64_t key = keys[i];
        const int bin = thr >= (uint32_t)NBINS ? 0 : score_bin(key_score(key), U);
        if (thr >= (uint32_t)NBINS || bin < (int)thr) {
            const int pos = atomicAdd(&s_nsel, 1);
            s_key[pos] = key;
            s_idx[pos] = (int32_t)i;
        } else if (bin == (int)thr) {
            const int pos = atomicAdd(&s_nbnd, 1);
            if (pos < BND_CAP) {
                s_bkey[pos] = key;
                s_bidx[pos] = (int32_t)i;
            }
        }
    }
    __syncthreads();
    int nsel = s_nsel;
    if (thr < (uint32_t)NBINS) {
        const int need = k - nsel;
        const int nb = s_nbnd;
        if (nb <= BND_CAP) {
            const int n2 = next_pow2(nb);
            for (int i = nb + tid; i < n2; i += SEL_THREADS) {
                s_bkey[i] = 0ull;
                s_bidx[i] = -1;
            }
            __syncthreads();
            bitonic_desc(s_bkey, s_bidx, n2);
            for (int i = tid; i < need; i += SEL_THREADS) {
                s_key[nsel + i] = s_bkey[i];
                s_idx[nsel + i] = s_bidx[i];
            }
        } else {
            // MSB-first radix select of the need-th best key of the bin.
            uint64_t prefix = 0, pmask = 0;
            int rem = need;
            for (int shift = 56; shift >= 0; shift -= 8) {
                for (int i = tid; i < 256; i += SEL_THREADS) s_cnt[i] = 0u;
                __syncthreads();
                for (uint32_t i = tid; i < N; i += SEL_THREADS) {
                    const uint64_t key = keys[i];
                    if (score_bin(key_score(key), U) == (int)thr && (key & pmask) == prefix)
                        atomicAdd(&s_cnt[(key >> shift) & 255u], 1u);
                }
                __syncthreads();
                if (tid == 0) {
                    uint32_t cum = 0;
                    for (int d = 255; d >= 0; --d) {
                        if (cum + s_cnt[d] >= (uint32_t)rem) {
                            s_digit = d;
                            s_rem = rem - (int)cum;
                            break;
                        }
                        cum += s_cnt[d];
                    }
                }
                __syncthreads();
                prefix |= (uint64_t)s_digit << shift;
                pmask |= 0xFFull << shift;
                rem = s_rem;
                __syncthreads();
            }
            for (uint32_t i = tid; i < N; i += SEL_THREADS) {
                const uint64_t key = keys[i];
                if (score_bin(key_score(key), U) == (int)thr && key >= prefix) {
                    const int pos = atomicAdd(&s_nsel, 1);
                    s_key[pos] = key;
                    s_idx[pos] = (int32_t)i;
                }
            }
        }
        nsel = k;
    }
    __syncthreads();
    const int n = nsel < k ? nsel : k;
    const int n2 = next_pow2(n > 0 ? n : 1);
    for (int i = n + tid; i < n2; i += SEL_THREADS) {
        s_key[i] = 0ull;
        s_idx[i] = -1;
    }
    __syncthreads();
    bitonic_desc(s_key, s_idx, n2);

    const int V = p.V, L = p.L, t = p.t;
    for (int j = tid; j < k; j += SEL_THREADS) {
        const size_t slot = (size_t)b * k + j;
        if (j < n) {
            const uint64_t key = s_key[j];
            const uint32_t f = key_flat(key);
            const int m = (int)(f / (uint32_t)V), v = (int)(f % (uint32_t)V);
            const int parent = b * p.M_in + m;
            p.parent_out[slot] = parent;
            p.token_out[slot] = v;
            p.node_out[slot] = p.schild[(size_t)b * p.cap + s_idx[j]];
            p.acc_out[slot] = key_score(key);
            if (p.tokens_out)
                for (int l = 0; l < L; ++l)
                    p.tokens_out[slot * L + l] =
                        l < t ? p.tokens_in[(size_t)parent * L + l] : (l == t ? v : -1);
            if (p.table_out)
                for (int l = 0; l < L; ++l)
                    p.table_out[slot * L + l] = l <= t ? p.table_in[(size_t)parent * L + l] : -1;
        } else {
            p.parent_out[slot] = -1;
            p.token_out[slot] = -1;
            p.node_out[slot] = -1;
            p.acc_out[slot] = -INFINITY;
            if (p.tokens_out)
                for (int l = 0; l < L; ++l) p.tokens_out[slot * L + l] = -1;
            if (p.table_out)
                for (int l = 0; l < L; ++l) p.table_out[slot * L + l] = -1;
        }
    }
}

}  // namespace

hipError_t launch_constrain_topk(const TrieDev &tr, const gr_tail_args &a, hipStream_t s) {
    TailParams p{};
    p.off = tr.node_offsets;
    p.child = tr.child_nodes;
    p.tok = tr.tokens;
    p.bmi = tr.bitmask_index;
    p.bli = tr.bloom_index;
    p.bm_tab = tr.bitmask_table;
    p.bl_tab = tr.bloom_table;
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
    p.ubound = (float *)(ws + ly.ubound);
    p.ctr = (uint32_t *)(ws + ly.ctr);
    p.hist = (uint32_t *)(ws + ly.hist);
    p.skey = (uint64_t *)(ws + ly.skey);
    p.schild = (int32_t *)(ws + ly.schild);
    p.cap = ly.cap;

    k_tail_prep<<<a.B, 256, 0, s>>>(p);
    dim3 g1((a.M_in + EXP_ROWS - 1) / EXP_ROWS, a.B);
    const size_t shm = sizeof(float) * EXP_WAVES * a.V;
    if (a.dtype == GR_BF16)
        k_expand<true><<<g1, EXP_THREADS, shm, s>>>(p);
    else
        k_expand<false><<<g1, EXP_THREADS, shm, s>>>(p);
    k_select<<<a.B, SEL_THREADS, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace gr
