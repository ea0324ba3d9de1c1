/*
 * gr.h -- C ABI of the wide-beam Semantic-ID decode step on AMD MI355X (gfx950).
 *
 * The decode step is the one of GRACE ("Generative Recommender Acceleration
 * Engine for Real-Time Ads Retrieval", arXiv 2608.00938): per SID position,
 *   (1) cross-attention with each request's beams stacked as the query
 *       sequence against that request's shared encoder context (Section 5.1,
 *       eqs 10-14, Appendix B);
 *   (2) self-attention over each beam's few generated tokens, read from a
 *       paged KV pool through a block table (Sections 3.3, 5.2, 5.3);
 *   (3) catalog-valid constrained decoding (CD, eq 1) plus Generative Target
 *       Matching (GTM, eqs 2-9) over a CSR trie with deduplicated bitmask and
 *       Bloom matcher rows (Section 4.4, Appendix A), full-vocabulary
 *       log-softmax, accumulated beam scores, per-request top-k and beam
 *       reorder (Sections 3.1 and 3.3).
 *
 * Conventions (every entry point):
 *   - Device pointers are owned by the caller; the library never frees them.
 *     Host pointers are read during the call only (copied where kept).
 *   - Hot-path calls (gr_cross_attn, gr_cross_attn_ws, gr_self_attn_paged,
 *     gr_joint_attn, gr_constrain_topk, gr_decode_step) never allocate and
 *     never synchronise the host: they validate, enqueue kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and return.  Scratch memory
 *     (the tail workspace, the split cross-attention workspace) is the
 *     caller's.
 *   - Argument errors return GR_E_INVALID / GR_E_UNSUPPORTED /
 *     GR_E_WORKSPACE before anything is launched; a failed launch returns
 *     GR_E_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation.  gr_last_error() gives a message (thread-local).
 *   - bf16 tensors hold raw bfloat16 bits (uint16 storage); outputs are
 *     rounded to nearest even from fp32 accumulators.
 *   - Row r of a beam tensor is request-major: r = b * M + m for request b,
 *     beam m (the flattening Appendix B assumes).
 *   - A trie handle is immutable after creation; calls on different streams
 *     may share it.
 */
#ifndef GR_H
#define GR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GR_OK = 0,
    GR_E_INVALID = -1,     /* bad pointer, shape, size or value                */
    GR_E_UNSUPPORTED = -2, /* valid request this build does not implement      */
    GR_E_NOMEM = -3,       /* host or device allocation failed (create/build)  */
    GR_E_WORKSPACE = -4,   /* workspace pointer null or smaller than required  */
    GR_E_HIP = -5          /* a HIP runtime call or kernel launch failed       */
} gr_status;

typedef enum { GR_F32 = 0, GR_BF16 = 1 } gr_dtype;

/* Message for the last non-OK status returned on this thread. */
const char *gr_last_error(void);
const char *gr_version(void);

/* ===================================================================== */
/* Index: the GTM SID trie (GRACE Section 4.4 and Appendix A).           */
/* ===================================================================== */

typedef struct gr_trie gr_trie;                 /* opaque, library-owned */
typedef struct gr_trie_builder gr_trie_builder; /* opaque, library-owned */

typedef struct {
    int32_t sid_length;  /* L: tokens per SID (1..16)                            */
    int32_t vocab_size;  /* V: codebook size per level (2..32768)                */
    int32_t w_bm;        /* uint64 words per bitmask matcher row (1..64)         */
    int32_t bloom_bits;  /* Bloom width w in bits: power of two in [64, 65536],  */
                         /* or 0 for a bitmask-only index                         */
    int32_t bloom_k;     /* hash probes per id (1..16); ignored if bloom_bits=0  */
    int32_t n_threads;   /* host threads used by the build (0 = all)             */
    int32_t keep_host;   /* 1: keep host copies of the arrays (gr_trie_view)     */
    int32_t host_only;   /* 1: keep host arrays only, no device copy (for         */
                         /* inspection; hot-path calls reject such a trie)       */
    int32_t bloom_slice_min; /* nodes with at least this many children also get */
                         /* a bit-sliced (column-major) copy of their children's */
                         /* Bloom and bitmask rows, which answers eqs 5 and 8   */
                         /* for all children at once (0: 48, -1: none); see      */
                         /* gr_trie_view.slice_words                             */
    /* k-way partitioned matchers (GRACE Section 4.2 and Figure 3; the      */
    /* modes of Section 6): each child entry keeps up to k partition unions */
    /* instead of one subtree union, and passes when one partition passes   */
    /* both the bitmask and the Bloom test.  The descendants of a node are  */
    /* its SIDs in ascending order; each goes to the partition whose union  */
    /* has the fewest set bits (bitmask and Bloom words together) after     */
    /* adding it, the lowest index on a tie; empty partitions are dropped.  */
    int32_t kway_mode;   /* 0: one union per entry (CD + GTM); 1: static, k =   */
                         /* kway_k[depth - 1]; 2: dynamic, k = 1, 2, ... until  */
                         /* the mean fill of the partitions is at most          */
                         /* kway_target_fill or k = kway_kmax                   */
    int32_t kway_k[16];  /* static: partitions per decoding position (>= 1)    */
    int32_t kway_kmax;   /* dynamic: largest k (>= 1)                           */
    float kway_target_fill; /* dynamic: fill target in (0, 1]                  */
} gr_trie_params;

/*
 * Start an index build from the catalog (GRACE Section 2.2 / Figure 1: the
 * trie is rebuilt offline from the ads stream).  `sids` [n_sids, L] int32 host
 * array of catalog SIDs, tokens in [0, V); a SID listed twice is the same SID.
 * L * ceil(log2 V) must be <= 64.  Returns GR_E_INVALID on a bad token or
 * parameter, GR_E_NOMEM if host memory runs out.
 */
gr_status gr_trie_builder_create(const gr_trie_params *params, const int32_t *sids,
                                 int64_t n_sids, gr_trie_builder **out);

/*
 * Add ads (may be called repeatedly, in any order, to stream large catalogs).
 *   ad_sid      [n_ads] int64: catalog row of the SID the ad belongs to
 *   rules       [n_ads, w_bm] uint64: the ad's targeting bitmask (eq 4 input)
 *   geo_offsets [n_ads + 1] int64: ad a's geo allow-list is
 *               geo_ids[geo_offsets[a] .. geo_offsets[a+1]) (ignored and may be
 *               NULL for a bitmask-only index)
 *   geo_ids     int32 geo ids (>= 0)
 * The ad's Bloom filter is the OR of bloom(id) over its list, with
 * bloom(id) = the bloom_k positions of gr_bloom_probes (eqs 8-9 input).
 * All host arrays; GR_E_INVALID on an out-of-range SID row or geo id < 0.
 */
gr_status gr_trie_builder_add_ads(gr_trie_builder *b, int64_t n_ads,
                                  const int64_t *ad_sid, const uint64_t *rules,
                                  const int64_t *geo_offsets, const int32_t *geo_ids);

/*
 * Finish: build the CSR trie (nodes numbered breadth-first, children of a
 * node sorted by token), the matcher rows of every non-root node as the OR of
 * its subtree's ads (eqs 4 and 9), deduplicate identical rows, and upload
 * everything to the current HIP device.  Consumes and frees the builder
 * (also on error).  GR_E_NOMEM / GR_E_HIP on allocation or copy failure.
 */
gr_status gr_trie_builder_finish(gr_trie_builder *b, gr_trie **out);
void gr_trie_builder_destroy(gr_trie_builder *b);

/*
 * Appendix A layout (host side).  Used to create a trie from arrays the
 * caller built (gr_trie_create) and to inspect a built one (gr_trie_view).
 * node_depth / node_parent / node_token are optional extras of the view
 * (NULL for gr_trie_create): depth of each node, its parent (-1 for the
 * root) and the token on the edge into it (-1 for the root).
 */
typedef struct {
    int32_t vocab_size, sid_length, w_bm, bloom_bits, bloom_k;
    int64_t num_nodes, num_entries, bm_rows, bl_rows;
    const int32_t *node_offsets;   /* [num_nodes + 1]                            */
    const int32_t *child_nodes;    /* [num_entries]                              */
    const int16_t *tokens;         /* [num_entries]                              */
    const int32_t *bitmask_index;  /* [num_entries] row of bitmask_table         */
    const int32_t *bloom_index;    /* [num_entries] row of bloom_table (or NULL) */
    const uint64_t *bitmask_table; /* [bm_rows, w_bm]                            */
    const uint64_t *bloom_table;   /* [bl_rows, bloom_bits / 64] (or NULL)       */
    const int32_t *node_depth;     /* [num_nodes] (view only)                    */
    const int32_t *node_parent;    /* [num_nodes] (view only)                    */
    const int16_t *node_token;     /* [num_nodes] (view only)                    */
    int64_t slice_words;           /* 8-byte words of bit-sliced matcher blocks   */
                                   /* on the device (info only)                   */
    /* k-way partitioned matchers (NULL / 0 without them): entry e's       */
    /* partitions are kway_bitmask_index / kway_bloom_index [kway_offsets[e] */
    /* .. kway_offsets[e + 1]), rows of the same deduplicated tables.       */
    const int32_t *kway_offsets;   /* [num_entries + 1]                           */
    const int32_t *kway_bitmask_index; /* [kway_rows]                             */
    const int32_t *kway_bloom_index;   /* [kway_rows] (or NULL)                   */
    int64_t kway_rows;
} gr_trie_view;

/*
 * Upload caller-built Appendix A arrays (host) to the current device.
 * Validates: offsets non-decreasing from 0 to num_entries, child ids in
 * [1, num_nodes), tokens in [0, V), matcher ids in range, tokens of one node
 * strictly increasing.  GR_E_INVALID names the first violation.
 * Nodes with at least 48 children also get the bit-sliced copy described at
 * gr_trie_params.bloom_slice_min.
 */
gr_status gr_trie_create(const gr_trie_view *arrays, gr_trie **out);

/* Host copies of a trie built with keep_host = 1 (GR_E_INVALID otherwise).
 * The pointers stay valid until gr_trie_destroy. */
gr_status gr_trie_host_view(const gr_trie *t, gr_trie_view *out);

/* Sizes of a trie (any trie). */
gr_status gr_trie_info(const gr_trie *t, gr_trie_view *out_sizes_only);
void gr_trie_destroy(gr_trie *t);

/*
 * Bloom probe positions of geo ids (GRACE Section 4.3: bloom(l) of a user
 * location; the pages fix no hash family): h = first SplitMix64 output from
 * state id, h1 = low 32 bits, h2 = high 32 bits | 1, position i =
 * (h1 + i * h2) mod bloom_bits for i < bloom_k.  Host arrays:
 * ids [n] -> positions [n, bloom_k].  Used to encode each request's
 * N_loc locations for gr_constrain_topk.
 */
gr_status gr_bloom_probes(const int32_t *ids, int64_t n, int32_t bloom_bits,
                          int32_t bloom_k, uint32_t *positions);

/* ===================================================================== */
/* A1: cross-attention, beam-as-query (GRACE Section 5.1, eqs 11-14).     */
/* ===================================================================== */
/*
 * out[b*M+m, h, :] = softmax_tau(q[b*M+m,h,:] . k_ctx[b,h,tau,:] / sqrt(d_h))
 *                    @ v_ctx[b,h,:,:]
 * q, out [B*M, H, d_h]; k_ctx, v_ctx [B, H, T_ctx, d_h]; all device, dense,
 * row-major, dtype `dtype` (bf16: MFMA path, fp32 accumulation; f32: fp32
 * path).  No mask: every context token is valid.
 * Limits: bf16 needs d_h in {32, 64, 128}; f32 needs d_h <= 64; both need
 * B, M, H, T_ctx >= 1.  bf16 also needs one request's queries
 * (M*H*d_h*2 bytes) and one head's context (T_ctx*d_h*2 bytes) below 2^32
 * bytes (they are read through 32-bit buffer extents).
 * GR_E_INVALID / GR_E_UNSUPPORTED otherwise.
 */
gr_status gr_cross_attn(const void *q, const void *k_ctx, const void *v_ctx, void *out,
                        int32_t B, int32_t M, int32_t H, int32_t T_ctx, int32_t d_h,
                        gr_dtype dtype, void *stream);

/*
 * The same output, with the context split across workgroups when the launch
 * has few tiles (beams x heads x requests) and a long context: each split
 * runs the online softmax over its own key range and leaves its
 * unnormalised output, running max and normaliser in ws; a second launch
 * merges the splits with a log-sum-exp (the combination the GR-Inference
 * page uses to merge its context and beam parts).
 * gr_cross_attn_workspace returns the bytes ws must hold for these shapes
 * (0 when no split is used: f32, short contexts, or enough tiles).  ws is
 * caller-owned device memory, 16-byte aligned, holding no state between
 * calls; NULL runs gr_cross_attn.  GR_E_WORKSPACE if ws is given but
 * smaller than needed; otherwise the errors of gr_cross_attn.
 */
size_t gr_cross_attn_workspace(int32_t B, int32_t M, int32_t H, int32_t T_ctx, int32_t d_h,
                               gr_dtype dtype);
gr_status gr_cross_attn_ws(const void *q, const void *k_ctx, const void *v_ctx, void *out,
                           int32_t B, int32_t M, int32_t H, int32_t T_ctx, int32_t d_h,
                           gr_dtype dtype, void *ws, size_t ws_bytes, void *stream);

/* ===================================================================== */
/* A2: paged short-prefix self-attention (GRACE Sections 3.3, 5.2, 5.3). */
/* ===================================================================== */
/*
 * At step t for rows i < R:
 *   k_pool[f] = k_new[i], v_pool[f] = v_new[i], table[i*L + t] = f,
 *     with f = fresh_base + i (one block = one token of one row, all heads);
 *   out[i,h,:] = softmax_j(q[i,h,:] . Kpool[table[i*L+j],h,:] / sqrt(d_h))
 *                @ Vpool[table[i*L+j],h,:]   over j = 0..t,
 *     skipping positions whose table entry is negative or not below
 *     pool_blocks (a dead row's missing past); each row sees only its own
 *     positions (the block-diagonal mask of Section 5.2).
 * q, k_new, v_new, out [R, H, d_h]; k_pool, v_pool [pool_blocks, H, d_h];
 * table [R, L] int32 (columns < t read, column t written).  Device, dtype.
 * GR_E_INVALID if fresh_base + R > pool_blocks, t >= L, or shapes are bad;
 * GR_E_UNSUPPORTED unless d_h = vec * 2^j <= 64 * vec (vec = 4 for bf16,
 * 2 for f32: a head's lanes form a power-of-two group) and
 * H * d_h <= 1024 * vec.
 */
gr_status gr_self_attn_paged(const void *q, const void *k_new, const void *v_new,
                             void *k_pool, void *v_pool, int64_t pool_blocks,
                             int32_t *table, int64_t fresh_base, int32_t R, int32_t t,
                             int32_t L, int32_t H, int32_t d_h, gr_dtype dtype,
                             void *out, void *stream);

/* ===================================================================== */
/* Joint attention: one softmax over the request's context and the row's */
/* own beam prefix (the shared-prefix beam attention of the Meituan       */
/* engine article; GR-Inference's GR-Decode-Attention, whose context and   */
/* beam parts are merged with a log-sum-exp, computes the same output).    */
/* ===================================================================== */
/*
 * For row r = b*M + m (R = B*M rows) and head h:
 *   out[r,h] = softmax_j(q[r,h] . key_j / sqrt(d_h)) . value_j over the keys
 *              k_ctx[b,h,0..T_ctx-1], then the row's prefix blocks
 *              k_pool[table[r,j],h] for j < t (a block id outside
 *              [0, pool_blocks) is skipped), then the current token k_new[r,h]
 *              (position t), with the matching values.
 * Like gr_self_attn_paged it writes k_new[r], v_new[r] to block
 * fresh_base + r of the pools and sets table[r, t] = fresh_base + r; the
 * prefix blocks it reads must lie outside [fresh_base, fresh_base + R).
 * Layouts: q, k_new, v_new, out [R, H, d_h]; k_ctx, v_ctx [B, H, T_ctx, d_h];
 * pools [pool_blocks, H, d_h]; table [R, L] int32 (L <= 16, 0 <= t < L).
 * bf16 (d_h in {32, 64, 128}, fp32 accumulation, context on MFMA) or fp32
 * (d_h <= 64).  All pointers are caller-owned device memory; no allocation,
 * no host synchronisation; argument errors return before any launch.
 */
gr_status gr_joint_attn(const void *q, const void *k_ctx, const void *v_ctx, const void *k_new,
                        const void *v_new, void *k_pool, void *v_pool, int64_t pool_blocks,
                        int32_t *block_table, int64_t fresh_base, int32_t B, int32_t M,
                        int32_t H, int32_t T_ctx, int32_t d_h, int32_t t, int32_t L,
                        gr_dtype dtype, void *out, void *stream);


/* ===================================================================== */
/* A3-A6: CD + GTM mask, log-softmax, scores, top-k, reorder.            */
/* ===================================================================== */
/*
 * For every row r (request b = r / M_in) with trie node node_in[r] >= 0:
 *   lse_r = log sum_v exp(x[r,v]) over ALL V logits (fp32);
 *   for each child entry j of the node (Appendix A Lookup):
 *     keep token v = tokens[j] iff
 *       (bitmask_table[bitmask_index[j]] & user_bm[b]) == user_bm[b]   (eq 5)
 *       and, with a Bloom matcher, some location l < n_loc of request b has
 *       all bloom_k probe bits user_probes[b,l,:] set in
 *       bloom_table[bloom_index[j]]                                   (eq 8)
 *   score[r,v] = acc_in[r] + (x[r,v] - lse_r)  (fp32) for kept v, else -inf.
 * Per request b, over flat index f = m*V + v of its M_in rows, the first
 * min(k_out, #finite) candidates in order (score desc, f asc) fill slots
 * s = b*k_out + j, sorted; the rest are dead:
 *   parent_out[s] = b*M_in + f/V, token_out[s] = f % V,
 *   node_out[s] = child node of that entry, acc_out[s] = score;
 *   dead: parent = token = node = -1, acc = -inf.
 * Reorder (optional, when tokens_out / table_out are non-NULL):
 *   tokens_out[s, 0..t-1] = tokens_in[parent, ..], tokens_out[s,t] = token,
 *   table_out[s, 0..t] = table_in[parent, 0..t]; other entries -1.
 * Rows with node_in < 0 (or not a node of the trie) are dead: no candidates.
 * Probe positions are taken modulo bloom_bits.
 * Limits: B <= 1024, V <= 4096, k_out <= 1024, M_in <= 65536,
 * M_in * V < 2^31, n_loc * (bloom_k rounded up to a multiple of 4) <= 2048,
 * w_bm <= 64, Bloom filters of at most 32768 bits (GR_E_UNSUPPORTED beyond).
 *
 * Workspace: device memory, 256-byte aligned, at least
 * gr_constrain_topk_workspace(B, M_in, V, k_out) bytes (GR_E_WORKSPACE
 * otherwise).  It must be zero-filled once before its first use (for
 * example with hipMemsetAsync); every completed call leaves it zero-filled
 * again, whatever the shapes of later calls.  Calls sharing a workspace must
 * be ordered (same stream).  A workspace that was not zero-filled gives
 * wrong selections, never an out-of-range access.
 *
 * The tail runs as two stages that can also be called one by one, in this
 * order, with the same arguments and workspace:
 *   gr_constrain      A3-A4: masks, log-softmax, scores; the survivors and
 *                     a score histogram go to the workspace (and dbg_mask /
 *                     dbg_scores when given);
 *   gr_topk_reorder   A5-A6: per-request top-k from the workspace, reorder,
 *                     all outputs.
 */
typedef struct {
    int32_t B, M_in, V, k_out, t, L, n_loc;
    gr_dtype dtype;                /* logits dtype                                  */
    const uint64_t *user_bm;       /* [B, w_bm]                                    */
    const uint32_t *user_probes;   /* [B, n_loc, bloom_k] (NULL if no Bloom)       */
    const void *logits;            /* [B*M_in, V]                                  */
    const int32_t *node_in;        /* [B*M_in]                                     */
    const float *acc_in;           /* [B*M_in]                                     */
    const int32_t *tokens_in;      /* [B*M_in, L] or NULL                          */
    const int32_t *table_in;       /* [B*M_in, L] or NULL                          */
    int32_t *parent_out;           /* [B*k_out]                                    */
    int32_t *token_out;            /* [B*k_out]                                    */
    int32_t *node_out;             /* [B*k_out]                                    */
    float *acc_out;                /* [B*k_out]                                    */
    int32_t *tokens_out;           /* [B*k_out, L] or NULL                         */
    int32_t *table_out;            /* [B*k_out, L] or NULL                         */
    uint64_t *dbg_mask;            /* [B*M_in, ceil(V/64)] or NULL: kept tokens    */
    float *dbg_scores;             /* [B*M_in, V] or NULL: score, -inf if masked   */
    void *ws;                      /* device workspace (gr_constrain_topk_workspace) */
    size_t ws_bytes;
} gr_tail_args;

size_t gr_constrain_topk_workspace(int32_t B, int32_t M_in, int32_t V, int32_t k_out);
/*
 * Launch shape of the tail for these sizes (informational; it sizes the
 * workspace): the constrain stage runs gx workgroups per request, workgroup
 * x taking the beam rows m = x + i * gx (i < rows_wg) and owning a survivor
 * segment of seg_cap entries; gx <= 2048.  Host pointers; GR_E_INVALID for
 * non-positive sizes or a NULL output.
 */
gr_status gr_constrain_topk_shape(int32_t B, int32_t M_in, int32_t V, int32_t *rows_wg,
                                  int32_t *gx, int64_t *seg_cap);
gr_status gr_constrain_topk(const gr_trie *trie, const gr_tail_args *args, void *stream);
/*
 * gr_constrain_topk without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and outputs,
 * with args->ws / ws_bytes ignored and the workspace taken from a scratch
 * array of 128 MiB that the library holds on each device it runs on, until
 * the process ends.  The call allocates nothing and frees nothing; it clears
 * the scratch's score histograms of the B requests with a kernel on
 * `stream`, then runs the tail.  Every call on one device shares that
 * device's scratch: calls that may overlap on one device (different streams,
 * threads or processes' graphs replayed concurrently) race and must be
 * ordered by the caller.  GR_E_UNSUPPORTED when the shapes need more than
 * 128 MiB (gr_constrain_topk_workspace(B, M_in, V, k_out) > 128 MiB, e.g.
 * B * M_in * V beyond about 8.9 M candidates); otherwise the errors of
 * gr_constrain_topk, with no GR_E_WORKSPACE.
 */
gr_status gr_constrain_topk_noalloc(const gr_trie *trie, const gr_tail_args *args,
                                    void *stream);
gr_status gr_constrain(const gr_trie *trie, const gr_tail_args *args, void *stream);
gr_status gr_topk_reorder(const gr_trie *trie, const gr_tail_args *args, void *stream);

/* ===================================================================== */
/* A7: one decode step = A1 -> A2 -> A3..A6 (GRACE Sections 3.1, 3.3).   */
/* ===================================================================== */
/*
 * Runs gr_cross_attn (rows B*M_in against k_ctx/v_ctx), gr_self_attn_paged
 * (fresh_base, pool, table = tail.table_in, which must be non-NULL) and
 * gr_constrain_topk (tail) on one stream.  The caller chains steps
 * t = 0..L-1 with M_0 = 1, M_{t+1} = k_t, fresh_base_t = sum_{s<t} B*M_s,
 * ping-ponging the state buffers (node/acc/tokens/table).  Outputs cross_out
 * and self_out [B*M_in, H, d_h] are written for every row.  The shape limits
 * of gr_cross_attn and gr_self_attn_paged both apply (GR_E_UNSUPPORTED).
 */
typedef struct {
    int32_t H, d_h, T_ctx;
    const void *k_ctx, *v_ctx;     /* [B, H, T_ctx, d_h]                            */
    const void *qx;                /* [B*M_in, H, d_h] cross-attention queries      */
    const void *q, *k_new, *v_new; /* [B*M_in, H, d_h] self-attention q/k/v         */
    void *k_pool, *v_pool;         /* [pool_blocks, H, d_h]                         */
    int64_t pool_blocks, fresh_base;
    void *cross_out, *self_out;    /* [B*M_in, H, d_h]                              */
    gr_tail_args tail;             /* dtype applies to every tensor of the step     */
    void *attn_ws;                 /* NULL, or the cross-attention workspace of     */
    size_t attn_ws_bytes;          /*   gr_cross_attn_ws (split context)            */
} gr_step_args;

gr_status gr_decode_step(const gr_trie *trie, const gr_step_args *args, void *stream);

/* ===================================================================== */
/* A whole decode as one HIP graph (GRACE Section 3.1: the decode loop is */
/* captured once and replayed, so the per-step launches cost no host      */
/* round trips).                                                           */
/* ===================================================================== */
/*
 * gr_decode_graph_create captures n_steps consecutive gr_decode_step calls
 * (steps[t] exactly as for gr_decode_step, t = 0..n_steps-1) issued on
 * `stream` into a HIP graph and instantiates it.  Nothing runs during
 * creation.  Every pointer in steps[] is baked into the graph: each launch
 * reads and writes exactly those caller-owned buffers, so the caller
 * refreshes inputs in place between launches and keeps the buffers alive
 * while the graph exists.  `stream` must be a created stream (not the
 * legacy default stream) that is not already capturing.  As for
 * gr_constrain_topk, the tail workspaces are zero-filled before the first
 * launch and every completed launch leaves them zeroed.
 * Errors: GR_E_INVALID for bad arguments (every step is validated as by
 * gr_decode_step, before anything is captured), GR_E_HIP when capture or
 * instantiation fails; *out is NULL then.  The graph owns no buffer;
 * gr_decode_graph_destroy frees the graph itself (NULL is a no-op).
 */
typedef struct gr_graph gr_graph;
gr_status gr_decode_graph_create(const gr_trie *trie, const gr_step_args *steps,
                                 int32_t n_steps, void *stream, gr_graph **out);
gr_status gr_decode_graph_launch(const gr_graph *graph, void *stream);
void gr_decode_graph_destroy(gr_graph *graph);

/* ===================================================================== */
/* Post stage (GRACE Section 2.1 steps 3-4, Section 2.2): the SID-to-ad    */
/* index expands finished SIDs into ads, and the exact ad-level matcher   */
/* (the ads targeting index) filters them.  Host memory and host threads, */
/* as the pages place this stage on the CPU.                               */
/* ===================================================================== */
/*
 * gr_ad_index_create takes the catalog (sids [n_sids, sid_length] int32,
 * distinct rows, tokens in [0, vocab_size)); gr_ad_index_add_ads appends
 * ads in id order (ad_sid [n] = catalog row, rules [n, w_bm] u64,
 * geo_offsets [n + 1] into geo_ids, as for gr_trie_builder_add_ads);
 * gr_ad_index_finish freezes it.  The index copies what it needs.
 *
 * gr_post_filter expands each row of tokens [n_rows, sid_length] (rows of
 * request b = r / rows_per_request; a row with a token outside [0, V), such
 * as a dead slot's -1, or a SID not in the catalog expands to nothing) and
 * tests every ad: it passes the bitmask part when each bit of
 * user_bm[b, :w_bm] is set in its rule words, the location part when one of
 * user_locs[b, :n_loc] is in its geo list (always, if n_loc = 0), and the
 * matcher when both do.  counts [n_rows, 4] int64 receive, per row: ads
 * expanded, bitmask passes, location passes, passes.  If pass_ids is not
 * NULL it receives the ids of the passing ads row by row (offsets = prefix
 * sums of counts[:, 3]); GR_E_WORKSPACE if they exceed pass_cap (counts are
 * still written).  n_threads <= 0: all hardware threads.
 */
typedef struct gr_ad_index gr_ad_index;
gr_status gr_ad_index_create(const int32_t *sids, int64_t n_sids, int32_t sid_length,
                             int32_t vocab_size, int32_t w_bm, gr_ad_index **out);
gr_status gr_ad_index_add_ads(gr_ad_index *index, int64_t n_ads, const int64_t *ad_sid,
                              const uint64_t *rules, const int64_t *geo_offsets,
                              const int32_t *geo_ids);
gr_status gr_ad_index_finish(gr_ad_index *index);
gr_status gr_post_filter(const gr_ad_index *index, const int32_t *tokens, int64_t n_rows,
                         int64_t rows_per_request, const uint64_t *user_bm,
                         const int32_t *user_locs, int32_t n_loc, int64_t *counts,
                         int64_t *pass_ids, int64_t pass_cap, int32_t n_threads);
void gr_ad_index_destroy(gr_ad_index *index);

#ifdef __cplusplus
}
#endif
#endif /* GR_H */
