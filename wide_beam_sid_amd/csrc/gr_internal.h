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
};

// Score histogram of the top-k pre-selection: NBINS bins of width
// 1 / BIN_SCALE nats below the best parent score of the request.
constexpr int NBINS = 4096;
constexpr float BIN_SCALE = 64.0f;
constexpr int MAX_V = 4096;          // vocabulary limit of the tail kernels
constexpr int MAX_K = 1024;          // top-k width limit (one slot per thread)
constexpr int MAX_PROBES = 2048;     // n_loc * bloom_k staged in LDS
constexpr int MAX_WBM = 64;

// Workspace carving of gr_constrain_topk (byte offsets).
struct TailWsLayout {
    size_t ubound, ctr, hist, skey, schild, total;
    int64_t cap;  // survivor capacity per request
};
TailWsLayout tail_ws_layout(int32_t B, int32_t M_in, int32_t V);

hipError_t launch_cross_attn(const void *q, const void *k, const void *v, void *out,
                             int B, int M, int H, int T, int d, gr_dtype dt,
                             hipStream_t s);
hipError_t launch_self_attn(const void *q, const void *k_new, const void *v_new,
                            void *k_pool, void *v_pool, int64_t pool_blocks, int32_t *table,
                            int64_t fresh_base, int R, int t, int L, int H, int d,
                            gr_dtype dt, void *out, hipStream_t s);
hipError_t launch_constrain_topk(const TrieDev &tr, const gr_tail_args &a,
                                 hipStream_t s);

}  // namespace gr
