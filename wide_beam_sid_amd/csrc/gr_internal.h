// Internal declarations shared by the host side (gr_host.cpp) and the HIP
// kernel translation units.  Not part of the public ABI (include/gr.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "../../include/gr.h"

namespace gr {

// Device copy of the Appendix A arrays of a GTM SID trie.
struct TrieDev {
    int32_t V, L, w_bm, w_bl, bloom_bits, bloom_k;
    int64_t num_nodes, num_entries, bm_rows, bl_rows;
    const int32_t *node_offsets;
    const int32_t *child_nodes;
    const int16_t *tokens;
    const int32_t *bitmask_index;
    const int32_t *bloom_index;
    const uint64_t *bitmask_table;
    const uint64_t *bloom_table;
    // Bit-sliced matcher blocks of wide nodes: node_slice[n] is the word
    // offset of node n's block in slice_table (-1: none).  The block holds,
    // for each matcher bit position pos (bloom_bits Bloom positions if there
    // is a Bloom matcher, then 64 * w_bm bitmask positions), ceil(c / 64)
    // words whose bit j is bit pos of the row of the node's j-th child entry.
    const int64_t *node_slice;
    const uint64_t *slice_table;
    int64_t slice_words;
    // Each child entry's bitmask row in entry order ([num_entries, w_bm];
    // null when w_bm > ENTRY_BM_MAX_W): one contiguous read with the entry
    // instead of a dependent gather through bitmask_index.
    const uint64_t *entry_bitmask;
    // k-way partitioned matchers (null without them): entry e's partitions
    // are kway_bmi / kway_bli [kway_offsets[e], kway_offsets[e + 1]).
    const int32_t *kway_offsets;
    const int32_t *kway_bmi;
    const int32_t *kway_bli;
    int64_t kway_rows;
    // The root's children are nodes 1..n_root in token order (0 otherwise):
    // then a step after the root can take its rows node-major.
    int32_t n_root;
};
constexpr int ENTRY_BM_MAX_W = 2;

// Score histogram of the top-k pre-selection: NBINS bins of width
// 1 / BIN_SCALE nats below the best parent score of the request.
constexpr int NBINS = 2048;
constexpr float BIN_SCALE = 32.0f;
constexpr int MAX_V = 4096;          // vocabulary limit of the tail kernels
constexpr int MAX_K = 1024;          // top-k width limit (one slot per thread)
constexpr int MAX_PROBES = 2048;     // n_loc * bloom_k staged in LDS
constexpr int MAX_WBM = 64;

constexpr int MAX_ROWS_WG = 32;      // beam rows per expand workgroup (upper bound)

// Launch shape of the expand kernel: workgroup x of request b takes rows
// m = x + i * gx (i < rows_wg) and owns a survivor segment of seg_cap
// entries (a row has at most V children), so no segment can overflow.  A
// segment's count is padded to a multiple of 8 with zero keys (never a real
// key) whose bin is 0xFFFF (never a real bin).
struct TailShape {
    int rows_wg, gx;
    int64_t seg_cap;
};
constexpr int MAX_M_IN = 65536;      // beam rows per request entering the tail
constexpr int MAX_B = 1024;          // requests per tail call (histogram region)
constexpr int MAX_GX = 2048;         // expand workgroups per request
constexpr int NM_MAX_GX = 1024;      // expand workgroups per request with a node-major pass
inline TailShape tail_shape(int32_t B, int32_t M_in, int32_t V) {
    const int64_t R = (int64_t)B * M_in;
    int64_t rw = R / 1024;
    const int64_t rw_min = ((int64_t)M_in + MAX_GX - 1) / MAX_GX;   // keeps gx <= MAX_GX
    if (rw < rw_min) rw = rw_min;
    rw = rw < 1 ? 1 : (rw > MAX_ROWS_WG ? MAX_ROWS_WG : rw);
    TailShape t;
    t.rows_wg = (int)rw;
    t.gx = (int)((M_in + rw - 1) / rw);
    // segments are read 8 bins / 2 keys at a time; a segment also holds up
    // to rows_wg rows' node-major survivors, each padded to a multiple of 8
    t.seg_cap = rw * (((int64_t)V + 7) & ~(int64_t)7);
    return t;
}

// Workspace carving of gr_constrain_topk (byte offsets).
// Per request, NCUT counters of survivors already counted in the histogram
// at or below cutoff bins cut_bin(j), j < NCUT_USED (the node-major pass
// drops candidates past the first cutoff that already holds k survivors).
// The cutoffs grow by about 2^(1/4): 15, 18, 21, 26, 31, 37, ..., 863, 1023
// (16 * 2^(j/4) with the quarter steps rounded to 76/64, 91/64, 108/64).
constexpr int NCUT = 32;
constexpr int NCUT_USED = 25;
__host__ __device__ constexpr int cut_bin(int j) {
    return ((16 << (j >> 2)) * ((j & 3) == 0 ? 64 : (j & 3) == 1 ? 76 : (j & 3) == 2 ? 91 : 108)) / 64 - 1;
}
struct TailWsLayout {
    size_t hist, segback, cut, inv, segcnt, skey, schild, sbin, total;
    TailShape shape;
};
TailWsLayout tail_ws_layout(int32_t B, int32_t M_in, int32_t V);

// Split-K plan of the bf16 cross-attention for a launch with few tiles and
// a long key loop: S splits of Ts keys (S = 1: no split) and the workspace
// bytes they need (S * B*M * H * (d + 2) floats).
struct CrossSplit {
    int S, Ts;
    size_t bytes;
};
CrossSplit cross_split_plan(int B, int M, int H, int T, int d, gr_dtype dt);
// The split tiles, then the log-sum-exp merge into out (bf16); ws holds
// pl.bytes, 16-byte aligned.
hipError_t launch_cross_split(const void *q, const void *k, const void *v, void *out, int B,
                              int M, int H, int T, int d, const CrossSplit &pl, void *ws,
                              hipStream_t s);
hipError_t launch_cross_attn(const void *q, const void *k, const void *v, void *out,
                             int B, int M, int H, int T, int d, gr_dtype dt,
                             hipStream_t s);
hipError_t launch_self_attn(const void *q, const void *k_new, const void *v_new,
                            void *k_pool, void *v_pool, int64_t pool_blocks, int32_t *table,
                            int64_t fresh_base, int R, int t, int L, int H, int d,
                            gr_dtype dt, void *out, hipStream_t s);
hipError_t launch_attn_pair(const void *qx, const void *k_ctx, const void *v_ctx, void *cross_out,
                            int B, int M, int H, int T, int d, const void *q, const void *k_new,
                            const void *v_new, void *k_pool, void *v_pool, int64_t pool_blocks,
                            int32_t *table, int64_t fresh_base, int t, int L, gr_dtype dt,
                            void *self_out, hipStream_t s);
hipError_t launch_joint_attn(const void *q, const void *k, const void *v, const void *k_new,
                             const void *v_new, void *k_pool, void *v_pool, int64_t pool_blocks,
                             int32_t *table, int64_t fresh_base, int B, int M, int H, int T, int d,
                             int t, int L, gr_dtype dt, void *out, hipStream_t s);
hipError_t launch_constrain(const TrieDev &tr, const gr_tail_args &a, hipStream_t s);

// Tail scratch held by the library (gr_constrain_topk_noalloc): the device
// address of this device's copy (looked up once per device), and a kernel
// that zero-fills the score histograms of B requests in a workspace.
constexpr size_t TAIL_SCRATCH_BYTES = (size_t)128 << 20;
hipError_t tail_scratch(void **out);
hipError_t launch_clear_hist(void *ws, int B, hipStream_t s);   // also the back counts

// Records msg as the message gr_last_error returns and returns st.
gr_status report(gr_status st, const char *msg);
hipError_t launch_topk_reorder(const TrieDev &tr, const gr_tail_args &a, hipStream_t s);
// Both halves, or, when every request enters with one row, one launch that
// does the whole tail.
hipError_t launch_tail(const TrieDev &tr, const gr_tail_args &a, hipStream_t s);

}  // namespace gr
